// Grouped (per-expert) columnwise NVFP4 for gfx950, optionally after a
// 16-point random Hadamard transform along the tokens of each 16-token block.
//
// Work unit: a workgroup (4 waves) owns 128 tokens x 256 columns of one group;
// wave w takes columns 64w .. 64w+63 of that range. Lane l holds columns
// 8 * (l / 8) .. +7 (16-byte loads) of the 16 tokens of token block l % 8, so
// the transform and the block amax of a column are entirely in-lane, and eight
// consecutive lanes write 64 contiguous code bytes of one plane row.
//
// The group of a workgroup is found on the device from the offsets: each lane of
// wave 0 takes one group, the padded lengths and tile counts are prefix-summed
// across the wave, and a ballot locates the group whose tile range holds the
// workgroup's slot. Workgroups past the last tile only take part in the
// arrival count. The grid is sized on the host for the largest possible number
// of tiles, (rows + 15 G) / 128 + G, since the offsets live on the device.
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
constexpr int kTileTok = 128;   // tokens per workgroup tile (8 blocks of 16)
constexpr int kTileCol = 256;   // columns per workgroup tile

struct GroupTile {
  int g;          // group index, or -1 when the slot holds no tile
  int tok0;       // first padded token of the tile within the group
  int n;          // real tokens of the group
  int pg;         // padded tokens of the group
  int row0;       // first row of the group in x
  int poff;       // first plane column of the group
  int mpad;       // total padded tokens (plane length)
  int tile0;      // first tile slot of the group
  int tiles;      // tile slots of the group
};

// Per-group layout, one group per lane of a wave (lanes >= groups hold empty
// groups): row range, padded length, tile count and their inclusive prefix sums
// across the wave. Offsets are clamped to [0, rows], so malformed device
// offsets cannot lead to reads outside x.
struct GroupScan {
  int lo, n, p, tiles, ps, ts;
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
  s.tiles = (s.p + kTileTok - 1) / kTileTok;
  s.ps = s.p;
  s.ts = s.tiles;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int a = __shfl_up(s.ps, o, 64), b = __shfl_up(s.ts, o, 64);
    if (lane >= o) {
      s.ps += a;
      s.ts += b;
    }
  }
  return s;
}

// Wave 0 locates the workgroup's tile; the result is shared through LDS.
__device__ GroupTile locate_tile(const int32_t* __restrict__ offsets, int groups, int rows, uint32_t slot) {
  __shared__ GroupTile s;
  if (threadIdx.x < 64) {
    const GroupScan q = group_scan(offsets, groups, rows);
    const int lane = threadIdx.x;
    const uint64_t before = __ballot(lane < groups && (uint32_t)q.ts <= slot);
    const int g = __popcll(before);
    const int gs = g < 64 ? g : 63;
    const int ts_g = __shfl(q.ts, gs, 64), tiles_g = __shfl(q.tiles, gs, 64);
    const int ps_g = __shfl(q.ps, gs, 64), p_g = __shfl(q.p, gs, 64);
    const int n_g = __shfl(q.n, gs, 64), lo_g = __shfl(q.lo, gs, 64);
    const int mpad = __shfl(q.ps, 63, 64);
    if (lane == 0) {
      GroupTile t;
      t.g = (g < groups) ? g : -1;
      t.tok0 = (int)(slot - (uint32_t)(ts_g - tiles_g)) * kTileTok;
      t.n = n_g;
      t.pg = p_g;
      t.row0 = lo_g;
      t.poff = ps_g - p_g;
      t.mpad = mpad;
      t.tile0 = ts_g - tiles_g;
      t.tiles = tiles_g;
      s = t;
    }
  }
  __syncthreads();
  return s;
}

// Workgroup (0, 0) of the encode pass, wave 0: padded offsets Poff[0] = 0,
// Poff[g + 1] = Poff[g] + 16 * ceil(n_g / 16), and each group's amax and S_dec
// (lane g reduces its group's partials: tile slots tile0 .. tile0 + tiles - 1
// of every column tile, `stride` slots apart).
// Max over the partials of tile slots tile0 .. tile0 + tiles - 1 of every
// column tile (all threads of the workgroup).
__device__ __forceinline__ float reduce_partials_2d(const Workspace* ws, uint32_t tile0, uint32_t tiles,
                                                    uint32_t stride, uint32_t coltiles) {
  float m = 0.0f;
  const uint32_t n = tiles * coltiles;
  for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
    const uint32_t y = i / tiles, k = i - y * tiles;
    m = fmaxf(m, ws->partial[y * stride + tile0 + k]);
  }
  return wg_max(m);
}

__device__ void report_groups(const int32_t* __restrict__ offsets, int groups, int rows, const Workspace* ws,
                              uint32_t stride, uint32_t coltiles, const float* amax_in, float* amax_out,
                              float* scale_out, int32_t* poff_out) {
  if (threadIdx.x >= 64) return;
  const GroupScan q = group_scan(offsets, groups, rows);
  const int lane = threadIdx.x;
  if (lane < groups) {
    float a = 0.0f;
    if (amax_in) {
      a = amax_in[lane];
    } else {
      const uint32_t t0 = (uint32_t)(q.ts - q.tiles);
      for (uint32_t y = 0; y < coltiles; ++y)
        for (int i = 0; i < q.tiles; ++i) a = fmaxf(a, ws->partial[y * stride + t0 + i]);
    }
    if (amax_out) amax_out[lane] = a;
    if (scale_out) scale_out[lane] = global_scale(a).dec;
    if (poff_out) poff_out[lane + 1] = q.ps;
  }
  if (lane == 0 && poff_out) poff_out[0] = 0;
}

// Load the lane's 16 tokens x 8 columns (zero for padding rows and columns
// past the end). A block with all 16 rows inside the group (every block but a
// group's last) takes unconditional loads from one base address with the row
// stride added as a scalar; only the last block pays per-row guards.
__device__ __forceinline__ void load_block(const uint16_t* __restrict__ x, int64_t ld_x, const GroupTile& t,
                                           uint32_t blk_tok0, uint32_t col, uint32_t cols, uint4 q[16]) {
  if ((int)blk_tok0 + 16 <= t.n && col < cols) {
    const uint16_t* p = x + (int64_t)(t.row0 + (int)blk_tok0) * ld_x + col;
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = *reinterpret_cast<const uint4*>(p + i * ld_x);
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int lt = (int)blk_tok0 + i;
      const bool ok = lt < t.n && col < cols;
      q[i] = ld16(x + (int64_t)(t.row0 + lt) * ld_x + col, ok);
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

// Pass 1: per-group amax of the (transformed, bf16-rounded) columnwise values.
template <bool RHT>
__global__ __launch_bounds__(kT) void k_grouped_amax(const uint16_t* __restrict__ x, int rows, uint32_t cols, int64_t ld_x,
                                                     const int32_t* __restrict__ offsets, int groups, uint32_t mask,
                                                     Workspace* ws, uint32_t gx, uint32_t gy, uint32_t chunk) {
  // work item = column tile * gx + tile slot, contiguous per XCD
  const uint32_t item = xcd_work_item(chunk);
  if (item >= gx * gy) return;
  const uint32_t slot = item % gx, ctile = item / gx;
  const GroupTile t = locate_tile(offsets, groups, rows, slot);
  const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  float m = 0.0f;
  if (t.g >= 0) {
    const uint32_t mb = lane & 7, cg = lane >> 3;
    const uint32_t col = ctile * kTileCol + wv * 64 + cg * 8;
    const uint32_t blk_tok0 = (uint32_t)t.tok0 + mb * 16;
    if ((int)blk_tok0 < t.pg) {
      uint4 q[16];
      load_block(x, ld_x, t, blk_tok0, col, cols, q);
      if constexpr (RHT) apply_signs(q, mask);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        float v[16];
        column(q, c, v);
        if constexpr (RHT) fwht16(v);
        m = fmaxf(m, fmaxf(max8_abs(v), max8_abs(v + 8)));
      }
      // max |bf16(0.25 y)| = bf16(0.25 max |y|): scaling by 0.25 and
      // round-to-nearest-even are both monotone.
      if constexpr (RHT) m = bf_lo(pack_bf16(m * 0.25f, 0.0f) & 0xFFFFu);
    }
  }
  publish_partial_at(ws, m, item);   // one slot per (token tile, column tile); 0 for slots past the last tile
}

// Pass 2: transform (optional), bf16 round-through, per-block scale and codes.
template <bool RHT, bool SR>
__global__ __launch_bounds__(kT) void k_grouped_quant(const uint16_t* __restrict__ x, int rows, uint32_t cols, int64_t ld_x,
                                                      const int32_t* __restrict__ offsets, int groups,
                                                      uint32_t mask, uint8_t* __restrict__ codes, int64_t ldc,
                                                      uint8_t* __restrict__ scales, int64_t lds,
                                                      const Workspace* ws, const float* amax_in, float* amax_out,
                                                      float* scale_out, int32_t* poff_out, uint64_t seed,
                                                      uint32_t offset, int64_t cap, uint32_t gx, uint32_t gy,
                                                      uint32_t chunk) {
  const uint32_t item = xcd_work_item(chunk);
  if (item >= gx * gy) return;
  const uint32_t slot = item % gx, ctile = item / gx;
  const GroupTile t = locate_tile(offsets, groups, rows, slot);
  __shared__ float rcp_tab[128];
  if (item == 0) report_groups(offsets, groups, rows, ws, gx, gy, amax_in, amax_out, scale_out, poff_out);
  if (t.g < 0) return;
  // this group's amax: its tile slots of every column tile of the amax pass
  const float amax = amax_in ? amax_in[t.g] : reduce_partials_2d(ws, (uint32_t)t.tile0, (uint32_t)t.tiles, gx, gy);
  const GScale g = global_scale(amax);
  fill_rcp_table(rcp_tab, g.dec);
  __syncthreads();
  const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint32_t mb = lane & 7, cg = lane >> 3;
  const uint32_t col = ctile * kTileCol + wv * 64 + cg * 8;
  const uint32_t blk_tok0 = (uint32_t)t.tok0 + mb * 16;
  if ((int)blk_tok0 >= t.pg || col >= cols) return;
  // Plane capacity guard: only malformed offsets can reach it.
  if ((int64_t)t.poff + blk_tok0 + 16 > cap) return;
  uint4 q[16];
  load_block(x, ld_x, t, blk_tok0, col, cols, q);
  if constexpr (RHT) apply_signs(q, mask);
  const uint32_t pcol = (uint32_t)t.poff + blk_tok0;      // plane column of the block's first token
  const uint64_t nbp = (uint64_t)(t.mpad >> 4);            // blocks per plane row
  // block index and addresses of column `col` once; the lane's next columns
  // differ by uniform strides (64-bit products cost several cycles)
  const uint64_t blk0 = (uint64_t)col * nbp + (pcol >> 4);
  uint8_t* cp = codes + (int64_t)col * ldc + (pcol >> 1);
  uint8_t* sp = scales + (int64_t)col * lds + (pcol >> 4);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float v[16];
    column(q, c, v);
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
    const uint32_t sc = block_scale(m, g.enc);
    const float rc = rcp_tab[sc];
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

template <bool RHT>
void launch_grouped_r(const GroupArgs& a, uint32_t gx, uint32_t gy, hipStream_t s) {
  const uint16_t* x = (const uint16_t*)a.x;
  const int64_t cap = a.ldc * 2 < a.lds * 16 ? a.ldc * 2 : a.lds * 16;
  const uint32_t chunk = xcd_chunk((uint64_t)gx * gy);
  const dim3 grid(xcd_grid((uint64_t)gx * gy));
  if (!a.amax_in)
    hipLaunchKernelGGL((k_grouped_amax<RHT>), grid, dim3(kT), 0, s, x, (int)a.rows, (uint32_t)a.cols, a.ld_x, a.offsets,
                       a.groups, a.mask, a.ws, gx, gy, chunk);
  if (a.sr)
    hipLaunchKernelGGL((k_grouped_quant<RHT, true>), grid, dim3(kT), 0, s, x, (int)a.rows, (uint32_t)a.cols, a.ld_x, a.offsets,
                       a.groups, a.mask, a.codes, a.ldc, a.scales, a.lds, a.ws, a.amax_in, a.amax_out,
                       a.scale_out, a.poff_out, a.seed, a.offset, cap, gx, gy, chunk);
  else
    hipLaunchKernelGGL((k_grouped_quant<RHT, false>), grid, dim3(kT), 0, s, x, (int)a.rows, (uint32_t)a.cols, a.ld_x,
                       a.offsets, a.groups, a.mask, a.codes, a.ldc, a.scales, a.lds, a.ws, a.amax_in,
                       a.amax_out, a.scale_out, a.poff_out, a.seed, a.offset, cap, gx, gy, chunk);
}

}  // namespace

// Tile slots x column tiles of the grid, which is also the number of partials
// the amax pass writes: the grid covers the largest possible number of tiles,
// (rows + 15 G) / 128 + G, since the offsets live on the device.
int64_t grouped_partials(int64_t rows, int64_t cols, int groups) {
  const int64_t max_tiles = (rows + 15 * (int64_t)groups + kTileTok - 1) / kTileTok + groups;
  return max_tiles * ((cols + kTileCol - 1) / kTileCol);
}

hipError_t launch_grouped(const GroupArgs& a, hipStream_t s) {
  const int64_t max_tiles = (a.rows + 15 * (int64_t)a.groups + kTileTok - 1) / kTileTok + a.groups;
  const uint32_t col_tiles = (uint32_t)((a.cols + kTileCol - 1) / kTileCol);
  if (a.rht) launch_grouped_r<true>(a, (uint32_t)max_tiles, col_tiles, s);
  else launch_grouped_r<false>(a, (uint32_t)max_tiles, col_tiles, s);
  return hipGetLastError();
}

}  // namespace nvfp4q
