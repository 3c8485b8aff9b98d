// 2D NVFP4 for gfx950: rowwise and columnwise (transposed) planes of one bf16
// tensor under one per-tensor scale, read once from HBM.
//
// One workgroup (512 threads) owns a 128 x 128 tile.
//  * Load: thread t reads one rowwise 16-element block (two adjacent 16-byte
//    loads) of rows t/8 + 64j, j = 0..1, so a wave reads 8 rows x 256 B per
//    instruction pair. The block's amax, scale and codes are computed in-lane;
//    rowwise codes leave as 8-byte stores, 64 contiguous bytes per row.
//  * The raw tile is staged in LDS (32 KiB) with the 16-byte chunk index of a
//    row XOR-ed by 4 * ((row / 16) mod 4), which spreads the eight 16-row
//    blocks a wave reads at one time over all banks.
//  * Columnwise: thread t owns columns 2 * (t / 8) .. +1 of rows
//    16 * (t % 8) .. +15 (16 LDS reads of 4 bytes), i.e. two columnwise blocks;
//    eight consecutive threads write 64 contiguous code bytes of one plane row.
//  * Several stacked weights (experts) in one launch: grid y is the expert;
//    each has its own amax and SR tags 2e (rowwise) and 2e + 1 (columnwise).
//  * 16 x 16 tile scales (NVFP4Q_SCALE_16X16): each wave's eight rows of a
//    16-row band meet in a lane shuffle per 16-column block, the two waves of
//    a band in LDS behind the staging barrier, and both planes encode with
//    the tile's scale.
// "[nvfp4_training] Optimize CuteDSL kernels for NVFP4 training", Optimization
// item 2 (the 2D weight kernel: wide shared-memory reads instead of 16-bit
// ones, paired columnwise reads sharing one amax and reciprocal) and item 5
// (scale bytes).
#include "rows.hpp"

namespace nvfp4q {

namespace {

constexpr int kTileR = 128, kTileC = 128;

__device__ __forceinline__ uint32_t swz_chunk(uint32_t chunk, uint32_t row) {
  return chunk ^ (((row >> 4) & 3u) << 2);
}

// T threads per tile: 128 / (T / 8) rows (rowwise) and 1024 / T columns
// (columnwise) per thread. TILE: one scale per 16 x 16 tile. DT: element type
// of x (bf16, fp16 or fp32; an fp32 tile stages 64 KiB).
// Tile order. Plain (gcols == 0): workgroup b takes tile b, row-major. Grouped
// by XCD (gcols = column count of 4 x 4 tile groups): the dispatcher sends
// workgroup b to XCD b mod 8, and the k-th workgroup of an XCD takes tile
// k mod 16 (row-major) of group 8 (k / 16) + b mod 8, so the 16 tiles of a
// 512 x 512 group run together on one XCD. Every 128-byte code line and every
// 32 bytes of a scale row that the group writes then come from one L2, where
// the pieces of neighbouring tiles merge before they leave it.
struct TileOrder {
  uint32_t tiles_r, tiles_c, gcols, ngroups;
};
__device__ __forceinline__ bool tile_of(const TileOrder o, uint32_t& tr, uint32_t& tc) {
  const uint32_t b = blockIdx.x;
  if (o.gcols == 0) {
    tr = b / o.tiles_c;
    tc = b - tr * o.tiles_c;
    return tr < o.tiles_r;
  }
  const uint32_t k = b / kXcds, gi = (k / 16) * kXcds + b % kXcds, u = k % 16;
  const uint32_t gr = gi / o.gcols, gc = gi - gr * o.gcols;
  tr = gr * 4 + u / 4;
  tc = gc * 4 + u % 4;
  return gi < o.ngroups && tr < o.tiles_r && tc < o.tiles_c;
}

template <int T, bool ROW, bool COL, bool SR, bool TILE, int DT>
__global__ __launch_bounds__(T) void k_quant_2d(const TwoDArgs a, const TileOrder order) {
  constexpr int kRpt = kTileR / (T / 8);  // rows per thread
  constexpr int kRs = T / 8;              // row stride between a thread's rows
  constexpr int kCpt = 1024 / T;          // columns per thread (columnwise)
  constexpr int kW = T / 64;              // waves; wave w holds rows 8w .. 8w + 7 (+ kRs j)
  constexpr int kEs = in_size<DT>();      // bytes per element
  constexpr int kRowBytes = kTileC * kEs; // per staged row
  constexpr int kPerChunk = 16 / kEs;     // elements per 16-byte chunk
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTileR * kRowBytes];
  __shared__ float rcp_tab[128];
  // TILE: maximum of each wave's 8 rows of every 16-column block, per row slot j
  __shared__ float part[TILE ? kRpt : 1][TILE ? kW : 1][8];
  const uint32_t e = blockIdx.y;  // expert
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const int64_t ld_x = a.ld_x;
  const int64_t rldc = a.rldc, rlds = a.rlds, cldc = a.cldc, clds = a.clds;
  const char* __restrict__ x = (const char*)a.x + (int64_t)e * rows * ld_x * kEs;
  uint8_t* __restrict__ rcodes = ROW ? a.rcodes + (int64_t)e * rows * rldc : nullptr;
  uint8_t* __restrict__ rscales = ROW ? a.rscales + (int64_t)e * rows * rlds : nullptr;
  uint8_t* __restrict__ ccodes = COL ? a.ccodes + (int64_t)e * cols * cldc : nullptr;
  uint8_t* __restrict__ cscales = COL ? a.cscales + (int64_t)e * cols * clds : nullptr;
  const uint64_t seed = a.seed;
  const uint32_t offset = a.offset;
  const uint32_t t = threadIdx.x;
  uint32_t tr, tc;
  if (!tile_of(order, tr, tc)) return;  // idle: no barrier or partial depends on it
  const uint32_t row0 = tr * kTileR, col0 = tc * kTileC;

  // ---- load kRpt rows x one 16-element block per thread
  const uint32_t bsub = t & 7, rsub = t >> 3;
  const uint32_t col = col0 + bsub * 16;
  Raw16<DT> q[kRpt];
  const char* xp = x + ((int64_t)(row0 + rsub) * ld_x + col) * kEs;
  if (row0 + kTileR <= rows && col0 + kTileC <= cols) {
    // a whole tile (all but the edge tiles): no guards, one base address
#pragma unroll
    for (int j = 0; j < kRpt; ++j)
#pragma unroll
      for (int l = 0; l < kEs; ++l)
        q[j].q[l] = *reinterpret_cast<const uint4*>(xp + (int64_t)(kRs * j) * ld_x * kEs + 16 * l);
  } else {
#pragma unroll
    for (int j = 0; j < kRpt; ++j) {
      const uint32_t r = row0 + rsub + kRs * j;
      const bool ok = r < rows && col < cols;
#pragma unroll
      for (int l = 0; l < kEs; ++l) q[j].q[l] = ld16(xp + (int64_t)(kRs * j) * ld_x * kEs + 16 * l, ok);
    }
  }
  const GScale g = consume_scales<T / 64>(a.ws, a.nparts, a.amax_in ? a.amax_in + e : nullptr,
                                          a.amax_out ? a.amax_out + e : nullptr,
                                          a.scale_out ? a.scale_out + e : nullptr, rcp_tab, e * a.nparts);
  if constexpr (COL) {
#pragma unroll
    for (int j = 0; j < kRpt; ++j) {
      const uint32_t lr = rsub + kRs * j;
#pragma unroll
      for (int h = 0; h < kEs; ++h)
        *reinterpret_cast<uint4*>(tile + lr * kRowBytes + swz_chunk(kEs * bsub + h, lr) * 16) = q[j].q[h];
    }
  }
  const uint32_t wid = t >> 6;
  if constexpr (TILE) {
    // lanes bsub + 8k, k = 0..7, hold the wave's 8 rows of block bsub
#pragma unroll
    for (int j = 0; j < kRpt; ++j) {
      float v[16];
      widen_raw16<DT>(q[j], v);
      float m = max16_abs(v);
      m = fmaxf(m, __shfl_xor(m, 8, 64));
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if ((t & 63) < 8) part[j][wid][t & 7] = m;
    }
    __syncthreads();  // also the staging barrier of the columnwise plane
  }
  // ---- rowwise plane from registers
  if constexpr (ROW) {
    // block index, code and scale addresses of row r0 once; rows 32 apart
    // then differ by uniform strides (64-bit products cost several cycles)
    const uint32_t nbr = cols >> 4;
    const uint32_t r0 = row0 + rsub;
    const uint64_t blk0 = (uint64_t)r0 * nbr + (col >> 4);
    uint8_t* cp = rcodes + (int64_t)r0 * rldc + (col >> 1);
    uint8_t* sp = rscales + (int64_t)r0 * rlds + (col >> 4);
#pragma unroll
    for (int j = 0; j < kRpt; ++j) {
      const uint32_t r = r0 + kRs * j;
      const bool ok = r < rows && col < cols;
      float v[16];
      widen_raw16<DT>(q[j], v);
      uint32_t sc;
      uint2 w;
      if constexpr (TILE) {
        // the row's 16-row band lies in waves 2 (wid / 2) and 2 (wid / 2) + 1
        const uint32_t w0 = wid & ~1u;
        sc = block_scale(fmaxf(part[j][w0][bsub], part[j][w0 + 1][bsub]), g.enc);
        w = encode_with_scale<SR>(v, sc, rcp_tab, blk0 + (uint64_t)(kRs * j) * nbr, seed, offset, 2 * e);
      } else {
        w = encode_block16<SR>(v, g, rcp_tab, sc, blk0 + (uint64_t)(kRs * j) * nbr, seed, offset, 2 * e);
      }
      if (ok) {
        *reinterpret_cast<uint2*>(cp + (int64_t)(kRs * j) * rldc) = w;
        sp[(int64_t)(kRs * j) * rlds] = (uint8_t)sc;
      }
    }
  }
  // ---- columnwise plane from the staged tile
  if constexpr (COL) {
    if constexpr (!TILE) __syncthreads();
    const uint32_t mb = t & 7, cg = t >> 3;           // 8 row blocks x T/8 column groups
    const uint32_t lc = cg * kCpt;                     // first local column
    const uint32_t cchunk = lc / kPerChunk;            // its 16-byte chunk of a staged row
    constexpr int kWords = kCpt * kEs / 4;             // 32-bit words of the thread's columns in one row
    uint32_t d[16][kWords];                            // 2-byte types: pairs of columns; fp32: one each
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t lr = mb * 16 + i;
      const uint8_t* src = tile + lr * kRowBytes + swz_chunk(cchunk, lr) * 16 + (lc % kPerChunk) * kEs;
      if constexpr (kWords == 4) {
        const uint4 u = *reinterpret_cast<const uint4*>(src);
        d[i][0] = u.x; d[i][1] = u.y; d[i][2] = u.z; d[i][3] = u.w;
      } else if constexpr (kWords == 2) {
        const uint2 u = *reinterpret_cast<const uint2*>(src);
        d[i][0] = u.x;
        d[i][1] = u.y;
      } else {
        d[i][0] = *reinterpret_cast<const uint32_t*>(src);
      }
    }
    const uint32_t grow = row0 + mb * 16;              // first row of the block
    const bool rok = grow < rows;
    const uint32_t nbc = rows >> 4;                    // column blocks per plane row
    const uint32_t gc0 = col0 + lc;
    const uint64_t cblk0 = (uint64_t)gc0 * nbc + (grow >> 4);
    uint8_t* ccp = ccodes + (int64_t)gc0 * cldc + (grow >> 1);
    uint8_t* csp = cscales + (int64_t)gc0 * clds + (grow >> 4);
    uint32_t tsc = 0;  // TILE: the scale of tile (band mb, column block lc / 16)
    if constexpr (TILE) {
      const uint32_t jj = (mb * 16) / kRs, w0 = (mb * 16 - jj * kRs) / 8;
      tsc = block_scale(fmaxf(part[jj][w0][lc >> 4], part[jj][w0 + 1][lc >> 4]), g.enc);
    }
#pragma unroll
    for (int c = 0; c < kCpt; ++c) {
      const uint32_t gc = gc0 + c;
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (DT == kInFP32) v[i] = __uint_as_float(d[i][c]);
        else if constexpr (DT == kInFP16) v[i] = (c & 1) ? h_hi(d[i][c >> 1]) : h_lo(d[i][c >> 1]);
        else v[i] = (c & 1) ? bf_hi(d[i][c >> 1]) : bf_lo(d[i][c >> 1]);
      }
      const uint32_t sc = TILE ? tsc : block_scale(max16_abs(v), g.enc);
      const float rc = rcp_tab[sc];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = v[i] * rc;
      uint2 out;
      if constexpr (SR) {
        U4 w = block_random(cblk0 + (uint64_t)c * nbc, 2 * e + 1, seed, offset);
        out.x = sr_pack8(v, w.x, w.y);
        out.y = sr_pack8(v + 8, w.z, w.w);
      } else {
        out.x = rtne_pack8(v);
        out.y = rtne_pack8(v + 8);
      }
      if (rok && gc < cols) {
        *reinterpret_cast<uint2*>(ccp + (int64_t)c * cldc) = out;
        csp[(int64_t)c * clds] = (uint8_t)sc;
      }
    }
  }
}

// NVFP4Q_2D_ORDER=0 selects the plain row-major tile order (for comparison);
// default: 4 x 4 tile groups per XCD.
bool order_2d() {
  static const bool v = [] {
    const char* e = getenv("NVFP4Q_2D_ORDER");
    return e == nullptr || atoi(e) != 0;
  }();
  return v;
}

template <int T, bool ROW, bool COL, bool TILE, int DT>
void launch_2d_t(const TwoDArgs& a, hipStream_t s) {
  TileOrder o;
  o.tiles_r = (uint32_t)((a.rows + kTileR - 1) / kTileR);
  o.tiles_c = (uint32_t)((a.cols + kTileC - 1) / kTileC);
  uint32_t wgs = o.tiles_r * o.tiles_c;
  o.gcols = 0;
  o.ngroups = 0;
  if (order_2d()) {
    o.gcols = (o.tiles_c + 3) / 4;
    o.ngroups = (o.tiles_r + 3) / 4 * o.gcols;
    wgs = (o.ngroups + kXcds - 1) / kXcds * kXcds * 16;
  }
  dim3 grid(wgs, a.experts), block(T);
  if (a.sr) hipLaunchKernelGGL((k_quant_2d<T, ROW, COL, true, TILE, DT>), grid, block, 0, s, a, o);
  else hipLaunchKernelGGL((k_quant_2d<T, ROW, COL, false, TILE, DT>), grid, block, 0, s, a, o);
}

// 512 threads per tile (two rows and two columns each): the tile's LDS
// limits a CU to four workgroups, which then hold 32 waves (256 threads: 16
// waves, 3 us slower on 8192 x 8192 with SR).
template <bool ROW, bool COL, int DT>
void launch_2d_rcd(const TwoDArgs& a, hipStream_t s) {
  if (a.tile16) launch_2d_t<512, ROW, COL, true, DT>(a, s);
  else launch_2d_t<512, ROW, COL, false, DT>(a, s);
}

template <bool ROW, bool COL>
void launch_2d_rc(const TwoDArgs& a, hipStream_t s) {
  if (a.dtype == kInFP16) launch_2d_rcd<ROW, COL, kInFP16>(a, s);
  else if (a.dtype == kInFP32) launch_2d_rcd<ROW, COL, kInFP32>(a, s);
  else launch_2d_rcd<ROW, COL, kInBF16>(a, s);
}

}  // namespace

hipError_t launch_quant_2d(const TwoDArgs& a, hipStream_t s) {
  const bool row = a.rcodes != nullptr, col = a.ccodes != nullptr;
  if (row && col) launch_2d_rc<true, true>(a, s);
  else if (row) launch_2d_rc<true, false>(a, s);
  else if (col) launch_2d_rc<false, true>(a, s);
  return hipGetLastError();
}

}  // namespace nvfp4q
