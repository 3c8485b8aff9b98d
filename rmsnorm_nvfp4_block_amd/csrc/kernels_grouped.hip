// Grouped (per-expert) columnwise NVFP4 for gfx950, optionally after a
// 16-point random Hadamard transform along the tokens of each 16-token block.
//
// Work unit: the padded token axis of all groups together is a sequence of
// 16-token blocks (group g occupies blocks Poff_g/16 .. Poff_{g+1}/16 - 1).
// A workgroup takes 8 consecutive blocks of that sequence and 256 columns;
// half-wave h of wave w takes block 2w + h, and lane l of the half takes
// columns 8l .. 8l+7 (16-byte loads of each of the block's 16 tokens), so the
// transform and the block amax of a column are in-lane and 32 lanes read 512
// contiguous bytes of a token row. Blocks run on across group boundaries, so
// no lane idles at a group's ragged end (with 128-token tiles inside each
// group, 18% of the lanes of the 16384 x 7168, 64-group workload idled); each
// half-wave finds its group by a ballot over the groups' block ranges, held
// one group per lane.
//
// Amax: the amax pass writes one partial maximum per (block, column tile);
// the encode pass reduces, for each group its wave touches, the partials of
// the group's blocks (contiguous slots). Per-group encode reciprocal tables
// live in LDS, two per wave.
//
// "[nvfp4_training] Optimize CuteDSL kernels for NVFP4 training": Grouped
// allocation tail (stop at the last padded row, leave the tail untouched);
// Config surface and AUTO (64 groups, device offsets); Fast math (the
// transform's bf16 round-through on the columnwise path); Optimization item 3
// (one Philox draw per 16-element block).
#include "device.hpp"
#include "launch.hpp"

namespace nvfp4q {

namespace {

constexpr int kT = 256;
constexpr int kTileCol = 256;      // columns per workgroup (32 lanes x 8)
constexpr int kBlocksPerWG = 8;    // token blocks per workgroup (2 per wave)

// Per-group layout, one group per lane of a wave (lanes >= groups hold empty
// groups): first row in x, real and padded length, and the inclusive prefix
// sum of the padded lengths. Offsets are clamped to [0, rows], so malformed
// device offsets cannot lead to reads outside x.
struct GroupScan {
  int lo, n, p, ps;
};
__device__ __forceinline__ GroupScan group_scan(const int32_t* __restrict__ offsets, int groups, int rows) {
  const int lane = threadIdx.x & 63;
  GroupScan s;
  s.lo = 0;
  s.n = 0;
  if (lane < groups) {
    s.lo = min(max(offsets[lane], 0), rows);
    s.n = min(max(offsets[lane + 1], s.lo), rows) - s.lo;
  }
  s.p = (s.n + 15) & ~15;
  s.ps = s.p;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(s.ps, o, 64);
    if (lane >= o) s.ps += a;
  }
  return s;
}

__device__ __forceinline__ int lane_int(int v, int g) { return __builtin_amdgcn_readlane(v, g); }

// One half-wave's block: its group and where its tokens are (wave-uniform).
struct Blk16 {
  int g;          // group
  int start;      // first padded token of the group (its first plane column)
  int n;          // real tokens of the group
  int row0;       // first row of the group in x
  bool valid;     // block inside the padded length of all groups, column inside cols
};

// The group holding padded token block tb (wave-uniform: every lane's test
// enters the ballot): the last group whose first padded token is <= 16 tb. Empty groups share their start with the next group, so
// counting every group that starts at or before the block gives it.
__device__ __forceinline__ Blk16 locate(const GroupScan& q, int groups, uint32_t tb, uint32_t mpad, uint32_t col,
                                        uint32_t cols) {
  const int lane = threadIdx.x & 63;
  const uint64_t bal = __ballot(lane < groups && (uint32_t)(q.ps - q.p) <= tb * 16u);
  const int g = (int)__popcll(bal) - 1;
  const int gs = g < 0 ? 0 : g;
  Blk16 b;
  b.g = gs;
  b.start = lane_int(q.ps - q.p, gs);
  b.n = lane_int(q.n, gs);
  b.row0 = lane_int(q.lo, gs);
  b.valid = tb * 16u < mpad && col < cols && g >= 0;
  return b;
}

// The lane's 16 tokens x 8 columns (zero for padding tokens). A block with all
// 16 tokens inside its group (every block but a group's last) takes
// unconditional loads from one base address with a scalar row stride.
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int64_t ld_x, const Blk16& b, uint32_t tb,
                                           uint32_t col, uint4 q[16]) {
  const int t0 = (int)(tb * 16u) - b.start;  // token of the block's first row within its group
  if (b.valid && t0 + 16 <= b.n) {
    const uint16_t* p = x + (int64_t)(b.row0 + t0) * ld_x + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = *reinterpret_cast<const uint4*>(p + i * ld_x);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = b.valid && t0 + i < b.n;
      q[i] = ld16(x + (int64_t)(b.row0 + t0 + i) * ld_x + col, ok);
    }
  }
}

// Column c (0..7) of the lane's 16 x 8 block as fp32.
__device__ __forceinline__ void column(const uint4 q[16], int c, float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = (c >> 1) == 0 ? q[i].x : (c >> 1) == 1 ? q[i].y : (c >> 1) == 2 ? q[i].z : q[i].w;
    v[i] = (c & 1) ? bf_hi(w) : bf_lo(w);
  }
}

// D: flips the sign of token row i of the lane's block where bit i of the
// mask is set. Row i's 16 bytes hold 8 bf16 columns, so one XOR with
// 0x80008000 per word flips all 8 (the bf16 sign bit becomes the fp32 sign
// bit when the value is widened). The mask is wave-uniform, so the per-row
// constants are scalar.
__device__ __forceinline__ void apply_signs(uint4 q[16], uint32_t mask) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t f = ((mask >> i) & 1u) ? 0x80008000u : 0u;
    q[i].x ^= f;
    q[i].y ^= f;
    q[i].z ^= f;
    q[i].w ^= f;
  }
}

// Four butterfly stages in Sylvester order on D v: for h = 1, 2, 4, 8 the
// pairs (i, i + h) with (i & h) == 0 become (a + b, a - b). The caller
// applies the 0.25 scaling.
__device__ __forceinline__ void fwht16(float v[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

// Max over the 32 lanes of each half-wave (all lanes take part).
__device__ __forceinline__ float half_wave_max(float m) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  return m;
}

// Geometry of one workgroup's work item (column tile, 8 blocks).
struct Work {
  uint32_t ctile;   // column tile
  uint32_t tb0;     // the wave's first block (half 0); tb0 + 1 is half 1's
  uint32_t tb;      // this lane's block
  uint32_t col;     // this lane's first column
};
__device__ __forceinline__ Work work_of(uint32_t item, uint32_t nwb) {
  Work w;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wid = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  w.ctile = item / nwb;
  w.tb0 = (item - w.ctile * nwb) * kBlocksPerWG + 2 * wid;
  w.tb = w.tb0 + (lane >> 5);
  w.col = w.ctile * kTileCol + (lane & 31) * 8;
  return w;
}

// Pass 1: per-(block, column tile) maximum of the (transformed, bf16-rounded)
// columnwise values, into partial[tb * ntc + ctile].
template <bool RHT>
__global__ __launch_bounds__(kT) void k_grouped_amax(const uint16_t* __restrict__ x, int rows, uint32_t cols,
                                                     int64_t ld_x, const int32_t* __restrict__ offsets, int groups,
                                                     uint32_t mask, Workspace* ws, uint32_t nwb, uint32_t ntiles,
                                                     uint32_t nb_max, uint32_t chunk) {
  const uint32_t item = xcd_work_item(chunk);
  if (item >= ntiles) return;
  const Work wk = work_of(item, nwb);
  const uint32_t ntc = ntiles / nwb;
  const GroupScan q = group_scan(offsets, groups, rows);
  const uint32_t mpad = (uint32_t)lane_int(q.ps, 63);
  // locate takes a wave-uniform block: the ballot reads every lane's test
  const Blk16 b0 = locate(q, groups, wk.tb0, mpad, wk.col, cols);
  const Blk16 b1 = locate(q, groups, wk.tb0 + 1, mpad, wk.col, cols);
  const Blk16 b = (threadIdx.x & 32) ? b1 : b0;
  float m = 0.0f;
  if (b.valid) {
    uint4 v16[16];
    load_block(x, ld_x, b, wk.tb, wk.col, v16);
    if constexpr (RHT) apply_signs(v16, mask);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      float v[16];
      column(v16, c, v);
      if constexpr (RHT) fwht16(v);
      m = fmaxf(m, fmaxf(max8_abs(v), max8_abs(v + 8)));
    }
    // max |bf16(0.25 y)| = bf16(0.25 max |y|): scaling by 0.25 and
    // round-to-nearest-even are both monotone.
    if constexpr (RHT) m = bf_lo(pack_bf16(m * 0.25f, 0.0f) & 0xFFFFu);
  }
  m = half_wave_max(m);
  if ((threadIdx.x & 31) == 0 && wk.tb < nb_max) ws->partial[wk.tb * ntc + wk.ctile] = m;
}

// Amax of group g (wave-uniform): the partials of its blocks over every
// column tile (contiguous slots), reduced by the whole wave, four loads in
// flight per lane. Slots stop at lim, the slots the amax pass writes (only
// malformed offsets can reach past it).
__device__ __forceinline__ float group_amax(const Workspace* ws, const GroupScan& q, int g, uint32_t ntc,
                                            uint32_t lim) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t lo = min(((uint32_t)lane_int(q.ps - q.p, g) >> 4) * ntc, lim);
  const uint32_t n = min(((uint32_t)lane_int(q.p, g) >> 4) * ntc, lim - lo);
  float m = 0.0f;
  for (uint32_t i = lane; i < n; i += 256) {
    float t[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) t[u] = i + 64 * u < n ? ws->partial[lo + i + 64 * u] : 0.0f;
    m = fmaxf(fmaxf(m, fmaxf(t[0], t[1])), fmaxf(t[2], t[3]));
  }
  return wave_max(m);
}

// Pass 2: transform (optional), bf16 round-through, per-block scale and codes.
template <bool RHT, bool SR>
__global__ __launch_bounds__(kT) void k_grouped_quant(const uint16_t* __restrict__ x, int rows, uint32_t cols,
                                                      int64_t ld_x, const int32_t* __restrict__ offsets, int groups,
                                                      uint32_t mask, uint8_t* __restrict__ codes, int64_t ldc,
                                                      uint8_t* __restrict__ scales, int64_t lds,
                                                      const Workspace* ws, const float* amax_in, float* amax_out,
                                                      float* scale_out, int32_t* poff_out, uint64_t seed,
                                                      uint32_t offset, int64_t cap, uint32_t nwb, uint32_t ntiles,
                                                      uint32_t nb_max, uint32_t chunk) {
  __shared__ float rcp_tab[kT / 64][2][128];  // per wave: the tables of its two blocks' groups
  const uint32_t item = xcd_work_item(chunk);
  if (item >= ntiles) return;
  const Work wk = work_of(item, nwb);
  const uint32_t ntc = ntiles / nwb;
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wid = threadIdx.x >> 6, half = lane >> 5;
  const GroupScan q = group_scan(offsets, groups, rows);
  const uint32_t mpad = (uint32_t)lane_int(q.ps, 63);
  // Workgroup 0, wave 0: padded offsets, and amax / S_dec of the groups no
  // encode wave reports (all of them with amax_in, else the empty ones).
  if (item == 0 && wid == 0 && lane < (uint32_t)groups) {
    if (amax_in != nullptr || q.p == 0) {
      const float a = amax_in ? amax_in[lane] : 0.0f;
      if (amax_out) amax_out[lane] = a;
      if (scale_out) scale_out[lane] = global_scale(a).dec;
    }
    if (poff_out) poff_out[lane + 1] = q.ps;
    if (lane == 0 && poff_out) poff_out[0] = 0;
  }
  // The wave's two blocks and their groups (wave-uniform).
  const Blk16 b0 = locate(q, groups, wk.tb0, mpad, wk.col, cols);
  const Blk16 b1 = locate(q, groups, wk.tb0 + 1, mpad, wk.col, cols);
  const Blk16 b = half ? b1 : b0;
  uint4 v16[16];
  load_block(x, ld_x, b, wk.tb, wk.col, v16);
  float a0, a1;
  if (amax_in) {
    a0 = amax_in[b0.g];
    a1 = amax_in[b1.g];
  } else {
    a0 = group_amax(ws, q, b0.g, ntc, nb_max * ntc);
    a1 = b1.g == b0.g ? a0 : group_amax(ws, q, b1.g, ntc, nb_max * ntc);
  }
  const GScale g0 = global_scale(a0), g1 = global_scale(a1);
  // The wave whose half holds a nonempty group's first block, in column tile
  // 0, reports that group's amax and S_dec.
  if (!amax_in && wk.ctile == 0 && lane == 0) {
    if (b0.valid && wk.tb0 * 16u == (uint32_t)b0.start) {
      if (amax_out) amax_out[b0.g] = a0;
      if (scale_out) scale_out[b0.g] = g0.dec;
    }
    if (b1.valid && (wk.tb0 + 1) * 16u == (uint32_t)b1.start) {
      if (amax_out) amax_out[b1.g] = a1;
      if (scale_out) scale_out[b1.g] = g1.dec;
    }
  }
  rcp_tab[wid][0][lane] = encode_mult(lane, g0.dec);
  rcp_tab[wid][0][lane + 64] = encode_mult(lane + 64, g0.dec);
  rcp_tab[wid][1][lane] = encode_mult(lane, g1.dec);
  rcp_tab[wid][1][lane + 64] = encode_mult(lane + 64, g1.dec);
  __syncthreads();
  if (!b.valid) return;
  const float* tab = rcp_tab[wid][half];
  const float enc = half ? g1.enc : g0.enc;
  const uint32_t pcol = wk.tb * 16u;                     // plane column of the block's first token
  // Plane capacity guard: only malformed offsets can reach it.
  if ((int64_t)pcol + 16 > cap) return;
  if constexpr (RHT) apply_signs(v16, mask);
  const uint64_t nbp = (uint64_t)(mpad >> 4);            // blocks per plane row
  // block index and addresses of column `col` once; the lane's next columns
  // differ by uniform strides (64-bit products cost several cycles)
  const uint64_t blk0 = (uint64_t)wk.col * nbp + (pcol >> 4);
  uint8_t* cp = codes + (int64_t)wk.col * ldc + (pcol >> 1);
  uint8_t* sp = scales + (int64_t)wk.col * lds + (pcol >> 4);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v[16];
    column(v16, c, v);
    if constexpr (RHT) {
      fwht16(v);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const uint32_t p = pack_bf16(v[i] * 0.25f, v[i + 1] * 0.25f);
        v[i] = bf_lo(p);
        v[i + 1] = bf_hi(p);
      }
    }
    const float m = fmaxf(max8_abs(v), max8_abs(v + 8));
    const uint32_t sc = block_scale(m, enc);
    const float rc = tab[sc];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = v[i] * rc;
    uint2 out;
    if constexpr (SR) {
      const U4 w = block_random(blk0 + (uint64_t)c * nbp, 1, seed, offset);
      out.x = sr_pack8(v, w.x, w.y);
      out.y = sr_pack8(v + 8, w.z, w.w);
    } else {
      out.x = rtne_pack8(v);
      out.y = rtne_pack8(v + 8);
    }
    *reinterpret_cast<uint2*>(cp + (int64_t)c * ldc) = out;
    sp[(int64_t)c * lds] = (uint8_t)sc;
  }
}

// Upper bound of the padded token blocks of all groups:
// sum ceil(n_g / 16) <= (rows + 15 G) / 16.
int64_t grouped_blocks(int64_t rows, int groups) { return (rows + 15 * (int64_t)groups) / 16; }

template <bool RHT>
void launch_grouped_r(const GroupArgs& a, hipStream_t s) {
  const uint16_t* x = (const uint16_t*)a.x;
  const int64_t cap = a.ldc * 2 < a.lds * 16 ? a.ldc * 2 : a.lds * 16;
  const uint32_t nb_max = (uint32_t)grouped_blocks(a.rows, a.groups);
  const uint32_t nwb = (nb_max + kBlocksPerWG - 1) / kBlocksPerWG < 1 ? 1 : (nb_max + kBlocksPerWG - 1) / kBlocksPerWG;
  const uint32_t ntc = (uint32_t)((a.cols + kTileCol - 1) / kTileCol);
  const uint32_t ntiles = nwb * ntc;  // work items: column tile major, blocks contiguous per XCD
  const uint32_t chunk = xcd_chunk(ntiles);
  const dim3 grid(xcd_grid(ntiles));
  if (!a.amax_in)
    hipLaunchKernelGGL((k_grouped_amax<RHT>), grid, dim3(kT), 0, s, x, (int)a.rows, (uint32_t)a.cols, a.ld_x,
                       a.offsets, a.groups, a.mask, a.ws, nwb, ntiles, nb_max, chunk);
  if (a.sr)
    hipLaunchKernelGGL((k_grouped_quant<RHT, true>), grid, dim3(kT), 0, s, x, (int)a.rows, (uint32_t)a.cols, a.ld_x,
                       a.offsets, a.groups, a.mask, a.codes, a.ldc, a.scales, a.lds, a.ws, a.amax_in, a.amax_out,
                       a.scale_out, a.poff_out, a.seed, a.offset, cap, nwb, ntiles, nb_max, chunk);
  else
    hipLaunchKernelGGL((k_grouped_quant<RHT, false>), grid, dim3(kT), 0, s, x, (int)a.rows, (uint32_t)a.cols,
                       a.ld_x, a.offsets, a.groups, a.mask, a.codes, a.ldc, a.scales, a.lds, a.ws, a.amax_in,
                       a.amax_out, a.scale_out, a.poff_out, a.seed, a.offset, cap, nwb, ntiles, nb_max, chunk);
}

}  // namespace

// Partial slots of the amax pass: one per (padded token block, column tile).
int64_t grouped_partials(int64_t rows, int64_t cols, int groups) {
  return grouped_blocks(rows, groups) * ((cols + kTileCol - 1) / kTileCol);
}

hipError_t launch_grouped(const GroupArgs& a, hipStream_t s) {
  if (a.rht) launch_grouped_r<true>(a, s);
  else launch_grouped_r<false>(a, s);
  return hipGetLastError();
}

}  // namespace nvfp4q
