// Grouped (per-expert) columnwise NVFP4 for gfx950, optionally after a
// 16-point random Hadamard transform along the tokens of each 16-token block,
// and optionally the rowwise plane of the same rows (no transform, its own
// per-group amax) from the same loads.
//
// Work unit: the padded token axis of all groups together is a sequence of
// 16-token blocks (group g occupies blocks Poff_g/16 .. Poff_{g+1}/16 - 1).
// A wave takes a pair of consecutive blocks and a tile of 32 CPL columns:
// half-wave h takes block 2p + h of pair p, and lane l of the half takes
// columns CPL l .. CPL l + CPL - 1 (one 2 CPL-byte load per token row), so
// the transform and the block amax of a column are in-lane and 32 lanes read
// 64 CPL contiguous bytes of a token row. Blocks run on across group
// boundaries, so no lane idles at a group's ragged end; each half-wave finds
// its group by a ballot over the groups' block ranges, held one group per
// lane.
//
// Loads go through a buffer resource whose range ends with x; rows of a block
// past its group's end, and lanes without data, take an offset past the range
// and read zero without touching memory.
//
// Three kernels: the amax pass (a grid-stride loop of at most 1024
// workgroups) keeps the maximum of every group it meets in LDS and writes 64
// slots per workgroup and plane; a reduce kernel (one workgroup per group)
// takes each group's maximum over those slots; the encode pass reads one amax
// per group and plane, keeps per-group encode reciprocal tables in LDS (two
// per wave, written and read by that wave only), stages its codes and scales
// in LDS and writes them out in coalesced pieces of the transposed planes.
//
// "[nvfp4_training] Optimize CuteDSL kernels for NVFP4 training": Grouped
// allocation tail (stop at the last padded row, leave the tail untouched);
// Config surface and AUTO (64 groups, device offsets); Fast math (the
// transform's bf16 round-through on the columnwise path); Optimization item 3
// (one Philox draw per 16-element block); Performance (the grouped row +
// column quantize).
#include "rows.hpp"

namespace nvfp4q {

namespace {

constexpr int kT = 256;
constexpr int kWaves = kT / 64;

// Buffer loads: byte offsets at or past kOutOfRange are never in range.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Workspace slots of the per-group amax written by the reduce kernel (after
// the amax pass's partials): columnwise, then rowwise.
constexpr int kGroupAmax = kPartials - 128;
constexpr int kGroupAmaxRow = kPartials - 64;

// Per-group layout, one group per lane of a wave (lanes >= groups hold empty
// groups): first row in x, real and padded length, and the inclusive prefix
// sum of the padded lengths. Offsets are clamped to [0, rows], so malformed
// device offsets cannot lead to reads outside x.
struct GroupScan {
  int lo, n, p, ps;
};
// Inclusive prefix sum over the 64 lanes by DPP: shifts by 1, 2, 4 and 8
// within each 16-lane row (lanes shifted in from outside the row add 0), then
// each row adds the totals of the rows before it through the row broadcasts
// (no LDS round trips, which a lane shuffle takes).
__device__ __forceinline__ int wave_prefix_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, kDppBcast15, 0xA, 0xF, false);  // row 0's total into row 1, row 2's into 3
  v += __builtin_amdgcn_update_dpp(0, v, kDppBcast31, 0xC, 0xF, false);  // rows 0-1's total into rows 2 and 3
  return v;
}
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
  s.ps = wave_prefix_sum(s.p);
  return s;
}

__device__ __forceinline__ int lane_int(int v, int g) { return __builtin_amdgcn_readlane(v, g); }

// One half-wave's block: its group and where its tokens are (wave-uniform).
struct Blk16 {
  int g;          // group
  int start;      // first padded token of the group (its first plane column)
  int n;          // real tokens of the group
  int row0;       // first row of the group in x
  bool valid;     // block inside the padded length of all groups
};

// The group holding padded token block tb (wave-uniform: every lane's test
// enters the ballot): the last group whose first padded token is <= 16 tb.
// Empty groups share their start with the next group, so counting every
// group that starts at or before the block gives it. A valid block holds at
// least one real token of its group.
__device__ __forceinline__ Blk16 locate(const GroupScan& q, int groups, uint32_t tb, uint32_t mpad) {
  const int lane = threadIdx.x & 63;
  const uint64_t bal = __ballot(lane < groups && (uint32_t)(q.ps - q.p) <= tb * 16u);
  const int g = (int)__popcll(bal) - 1;
  const int gs = g < 0 ? 0 : g;
  Blk16 b;
  b.g = gs;
  b.start = lane_int(q.ps - q.p, gs);
  b.n = lane_int(q.n, gs);
  b.row0 = lane_int(q.lo, gs);
  b.valid = tb * 16u < mpad && g >= 0;
  return b;
}

// A buffer resource over x from row `row` to the end of x (record count
// capped below kOutOfRange).
template <int DT>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t x_from_row(const void* x, int64_t ld_x, int rows, int row) {
  int64_t left = ((int64_t)rows - row) * ld_x * in_size<DT>();
  left = left < 0 ? 0 : left > (int64_t)(kOutOfRange - 32) ? (int64_t)(kOutOfRange - 32) : left;
  return __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)x + (int64_t)row * ld_x * in_size<DT>()), (short)0,
                                           (int)left, 0x00020000);
}

// Work items: a workgroup takes 4 consecutive block pairs (wave w: pair
// 4 quad + w; half-wave h: block 2 pair + h) and one column tile of 32 CPL
// columns, so it writes 64 contiguous bytes of every plane row of its tile;
// block quads are the fast index, and workgroups are ordered XCD by XCD
// (xcd_work_item), so neighbouring quads, which fill the rest of those plane
// lines, run on the same L2.
struct Item {
  uint32_t ctile;   // column tile
  uint32_t tb0;     // the pair's first block (half 0); tb0 + 1 is half 1's
  Blk16 b0, b1;     // the two blocks' groups
  uint32_t tb;      // this lane's block
  uint32_t col;     // this lane's first column
  bool ok;          // this lane's block and columns hold data
};
// Workgroup item v (< nq * ntc), nq block quads: column tile and the wave's
// block pair (wave-uniform; may be past the last pair).
__device__ __forceinline__ void wg_item(uint32_t v, uint32_t nq, uint32_t& ctile, uint32_t& pair) {
  ctile = v / nq;
  pair = (v - ctile * nq) * kWaves + (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}
template <int CPL>
__device__ __forceinline__ Item item_of(uint32_t ctile, uint32_t pair, const GroupScan& q, int groups, uint32_t mpad,
                                        uint32_t cols) {
  Item it;
  const uint32_t lane = threadIdx.x & 63;
  it.ctile = ctile;
  it.tb0 = 2 * pair;
  it.b0 = locate(q, groups, it.tb0, mpad);
  it.b1 = locate(q, groups, it.tb0 + 1, mpad);
  it.tb = it.tb0 + (lane >> 5);
  it.col = it.ctile * (32 * CPL) + (lane & 31) * CPL;
  it.ok = ((lane >> 5) ? it.b1.valid : it.b0.valid) && it.col < cols;
  return it;
}

// The lane's 16 tokens x CPL columns of element type DT: 2-byte types as
// pairs (r[i][j] holds columns 2j, 2j + 1 of token row i), fp32 one per word.
template <int CPL, int DT>
using Tile = uint32_t[16][CPL * in_size<DT>() / 4];

// Issues the item's loads: one resource based at the first block's first row,
// row offsets in the per-lane offset (so the range check covers them).
template <int CPL, int DT>
__device__ __forceinline__ void load_item(const void* __restrict__ x, int64_t ld_x, int rows, const Item& it,
                                          bool live, Tile<CPL, DT>& r) {
  constexpr uint32_t kEs = in_size<DT>();
  constexpr int kBytes = CPL * kEs;  // per token row and lane: 8, 16 or 32
  const bool h = (threadIdx.x >> 5) & 1;
  // first row in x of each block: its group's row0 plus the block's first
  // token within the group
  const int t0a = (int)(it.tb0 * 16u) - it.b0.start, t0b = (int)((it.tb0 + 1) * 16u) - it.b1.start;
  const int ra = it.b0.valid ? it.b0.row0 + t0a : 0;
  const int rb = it.b1.row0 + t0b;
  const __amdgpu_buffer_rsrc_t rs = x_from_row<DT>(x, ld_x, rows, ra);
  const uint32_t ldb = (uint32_t)ld_x * kEs;
  // real tokens of the lane's block (none for an item that is only a refill
  // past the end of a run: its loads are issued but read nothing)
  const int left = live && it.ok ? (h ? it.b1.n - t0b : it.b0.n - t0a) : 0;
  const uint32_t v0 = (uint32_t)(h ? rb - ra : 0) * ldb + it.col * kEs;
  static_assert(CPL == 4 || CPL == 8, "4 or 8 columns per lane");
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t off = i < left ? v0 + (uint32_t)i * ldb : kOutOfRange;
    if constexpr (kBytes == 32) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u * hh, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j) r[i][4 * hh + j] = t[j];
      }
    } else if constexpr (kBytes == 16) {
      const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) r[i][j] = t[j];
    } else {
      const auto t = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
      r[i][0] = t[0];
      r[i][1] = t[1];
    }
  }
  // Every load of the item is issued before any of its data is used: left to
  // itself the scheduler moved the first uses in among the loads, and the waits
  // they need held the last loads back until the first had landed.
  __builtin_amdgcn_sched_barrier(0);
}

// Column c of the lane's tile as fp32.
template <int CPL, int DT>
__device__ __forceinline__ void column(const Tile<CPL, DT>& r, int c, float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if constexpr (DT == kInFP32) v[i] = __uint_as_float(r[i][c]);
    else if constexpr (DT == kInFP16) v[i] = (c & 1) ? h_hi(r[i][c >> 1]) : h_lo(r[i][c >> 1]);
    else v[i] = (c & 1) ? bf_hi(r[i][c >> 1]) : bf_lo(r[i][c >> 1]);
  }
}

// Column c of the lane's tile as fp32 with the transform's sign diagonal D
// applied: token row i changes sign where bit i of the mask is set. For bf16
// the flip rides on the widening: the low element is (w << 16) + 2^31 (adding
// 2^31 flips bit 31 alone), the high one (w & 0xFFFF0000) ^ 2^31 (one
// three-input logic instruction); fp16 and fp32 flip the widened word. The
// mask is wave-uniform, so the per-row constants are scalar.
template <int CPL, int DT>
__device__ __forceinline__ void column_signed(const Tile<CPL, DT>& r, int c, uint32_t mask, float v[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t s = ((mask >> i) & 1u) << 31;
    if constexpr (DT == kInBF16) {
      const uint32_t w = r[i][c >> 1];
      v[i] = (c & 1) ? __uint_as_float((w & 0xFFFF0000u) ^ s) : __uint_as_float((w << 16) + s);
    } else if constexpr (DT == kInFP32) {
      v[i] = __uint_as_float(r[i][c] ^ s);
    } else {
      const float h = (c & 1) ? h_hi(r[i][c >> 1]) : h_lo(r[i][c >> 1]);
      v[i] = __uint_as_float(__float_as_uint(h) ^ s);
    }
  }
}

// The transform's output rounded through the input's type (bf16, fp16; fp32:
// unchanged), two values at a time.
template <int DT>
__device__ __forceinline__ void round_through2(float& a, float& b) {
  if constexpr (DT == kInBF16) {
    a = bf16_round(a);
    b = bf16_round(b);
  } else if constexpr (DT == kInFP16) {
    a = (float)(_Float16)a;
    b = (float)(_Float16)b;
  }
}

// Butterfly stages in Sylvester order on D v: for h = 1, 2, 4, 8 (the
// first STAGES of them) the pairs (i, i + h) with (i & h) == 0 become
// (a + b, a - b). The caller applies the 0.25 scaling.
template <int STAGES = 4>
__device__ __forceinline__ void fwht16(float v[16]) {
#pragma unroll
  for (int h = 1; h < (1 << STAGES); h <<= 1) {
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

// Magnitude bits of the larger of two bf16 per half (sign bits cleared: for
// finite values the u16 order of |x| is the order of the magnitudes).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_mag(uint32_t acc, uint32_t w) {
  const u16x2 m = __builtin_elementwise_max(__builtin_bit_cast(u16x2, acc), __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu));
  return __builtin_bit_cast(uint32_t, m);
}

// Pass 1: per-group maxima. The launch has at most kAmaxGrid workgroups; each
// takes work items (4 block pairs x one column tile) in a grid-stride loop and
// keeps the maximum of every group it meets in LDS (non-negative floats
// compare like their bit patterns, so an LDS integer maximum suffices). At the
// end workgroup w writes its 64 group maxima into partial[w * 64 + g] (COL: of
// the transformed values, rounded through the input's type) and, for the
// rowwise plane (ROW: of |x| itself, no transform), into
// partial[rbase + w * 64 + g]; groups it never met get 0. The workspace thus
// holds grid x 64 slots per plane whatever the size of x.
constexpr int kAmaxGrid = 1024;
static_assert(2 * kAmaxGrid * 64 + 128 <= kPartials, "both planes' group maxima fit the workspace");

// One work item of the amax pass: the group maxima of the lane's blocks
// (columnwise: of the transform's output; rowwise: of |x|) into the
// workgroup's LDS slots gmc / gmr.
template <int CPL, bool RHT, bool FAST, bool COL, bool ROW, int DT>
__device__ __forceinline__ void amax_item(const Item& it, const Tile<CPL, DT>& r, uint32_t mask, uint32_t nb_max,
                                          uint32_t* gmc, uint32_t* gmr) {
  const uint32_t half = (threadIdx.x >> 5) & 1;
  // the half-wave's block and group (lane 0 of the half publishes)
  const bool writer = (threadIdx.x & 31) == 0 && it.tb < nb_max && (half ? it.b1.valid : it.b0.valid);
  const int g = half ? it.b1.g : it.b0.g;
  if constexpr (ROW) {
    float mr;
    if constexpr (DT == kInFP32) {
      uint32_t mm = 0;  // magnitude bits: their u32 order is the order of |x|
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < CPL; ++j) mm = max(mm, r[i][j] & 0x7FFFFFFFu);
      mr = __uint_as_float(mm);
    } else {
      uint32_t mm = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < CPL / 2; ++j) mm = pk_max_mag(mm, r[i][j]);
      const uint32_t hi = mm >> 16, lo = mm & 0xFFFFu, m16 = hi > lo ? hi : lo;
      mr = DT == kInBF16 ? __uint_as_float(m16 << 16) : h_lo(m16);
    }
    mr = half_wave_max(mr);  // lanes without data: 0
    if (writer) atomicMax(&gmr[g], __float_as_uint(mr));
  }
  if constexpr (COL) {
    float m = 0.0f;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      float v16[16];
      if constexpr (RHT) column_signed<CPL, DT>(r, c, mask, v16);
      else column<CPL, DT>(r, c, v16);
      if constexpr (RHT) {
        // The last stage only feeds the maximum: max(|RN(a + b)|, |RN(a - b)|)
        // = RN(|a| + |b|), since one of a + b, a - b has magnitude |a| + |b|,
        // the other at most that, and rounding is odd and monotone.
        fwht16<3>(v16);
        float s8[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) s8[i] = fabsf(v16[i]) + fabsf(v16[i + 8]);
        m = fmaxf(m, max8_abs(s8));
      } else {
        m = fmaxf(m, max16_abs(v16));
      }
    }
    // max |RN_T(0.25 y)| = RN_T(0.25 max |y|): scaling by 0.25 and
    // round-to-nearest-even are both monotone (fast math, fp32: no rounding).
    if constexpr (RHT) m = FAST ? m * 0.25f : round_t<DT>(m * 0.25f);
    m = half_wave_max(m);  // lanes without data hold zeros
    if (writer) atomicMax(&gmc[g], __float_as_uint(m));
  }
}

template <int CPL, bool RHT, bool FAST, bool COL, bool ROW, int DT>
__global__ __launch_bounds__(kT) void k_grouped_amax(const void* __restrict__ x, int rows, uint32_t cols,
                                                     int64_t ld_x, const int32_t* __restrict__ offsets, int groups,
                                                     uint32_t mask, Workspace* ws, uint32_t nq, uint32_t ntc,
                                                     uint32_t npairs, uint32_t nb_max, uint32_t rbase) {
  __shared__ uint32_t gmc[64], gmr[64];  // group maxima (fp32 bits) of this workgroup, columnwise / rowwise
  if (threadIdx.x < 64) {
    gmc[threadIdx.x] = 0u;
    gmr[threadIdx.x] = 0u;
  }
  __syncthreads();
  const GroupScan q = group_scan(offsets, groups, rows);
  const uint32_t mpad = (uint32_t)lane_int(q.ps, 63);
  const uint32_t nitems = nq * ntc, G = gridDim.x;
  // Item v's loads are issued into a tile (none read memory when the wave has
  // no block pair there); returns whether the wave has work in it.
  // Wave-uniform.
  auto fetch = [&](uint32_t v, Item& it, Tile<CPL, DT>& r) -> bool {
    uint32_t ctile = 0, pair = 0;
    if (v < nitems) wg_item(v, nq, ctile, pair);
    const bool live = v < nitems && pair < npairs;
    it = item_of<CPL>(ctile, pair, q, groups, mpad, cols);
    load_item<CPL, DT>(x, ld_x, rows, it, live, r);
    return live;
  };
  Tile<CPL, DT> r;
  Item it;
  for (uint32_t v = blockIdx.x; v < nitems; v += G)
    if (fetch(v, it, r)) amax_item<CPL, RHT, FAST, COL, ROW, DT>(it, r, mask, nb_max, gmc, gmr);
  __syncthreads();
  if (threadIdx.x < 64) {
    if (COL) ws->partial[blockIdx.x * 64 + threadIdx.x] = __uint_as_float(gmc[threadIdx.x]);
    if (ROW) ws->partial[rbase + blockIdx.x * 64 + threadIdx.x] = __uint_as_float(gmr[threadIdx.x]);
  }
}

// Between the passes, one workgroup per group: the maximum of the group's
// slots over the amax pass's workgroups (nwg of them), into the workspace for
// the encode pass and into amax_out / scale_out (rowwise: from rbase on, into
// ramax_out / rscale_out).
constexpr int kReduceThreads = 512;
template <bool COL, bool ROW>
__global__ __launch_bounds__(kReduceThreads) void k_grouped_reduce(Workspace* ws, uint32_t nwg, uint32_t rbase,
                                                                   float* amax_out, float* scale_out,
                                                                   float* ramax_out, float* rscale_out) {
  const int g = blockIdx.x;
  auto reduce = [&](const float* src) {
    float m = 0.0f;
    for (uint32_t w = threadIdx.x; w < nwg; w += kReduceThreads) m = fmaxf(m, src[w * 64 + g]);
    return wg_max<kReduceThreads / 64>(m);
  };
  if constexpr (COL) {
    const float m = reduce(ws->partial);
    if (threadIdx.x == 0) {
      ws->partial[kGroupAmax + g] = m;
      if (amax_out) amax_out[g] = m;
      if (scale_out) scale_out[g] = global_scale(m).dec;
    }
  }
  if constexpr (ROW) {
    const float m = reduce(ws->partial + rbase);
    if (threadIdx.x == 0) {
      ws->partial[kGroupAmaxRow + g] = m;
      if (ramax_out) ramax_out[g] = m;
      if (rscale_out) rscale_out[g] = global_scale(m).dec;
    }
  }
}

// Pass 2: transform (optional), bf16 round-through, per-block scale and codes.
// The group amax comes from amax_in, else from the reduce kernel.
//
// A work item is kItemBlocks consecutive blocks (wave w: pair
// kQuantWaves bg + w) of one column tile. Its codes and scales are staged in
// LDS and written out once the workgroup has encoded it: every plane row of
// the tile then receives 8 kItemBlocks code bytes and kItemBlocks scale bytes
// in single coalesced stores (written from the lanes that computed them, the
// pieces were 8 bytes and 1 byte, 8.7 KB apart, and those stores alone cost as
// much as the reads). Workgroups take items in XCD order (xcd_work_item), the
// blocks fastest, so the workgroups that complete a plane line share an L2.
// Measured on the 16384 x 7168, 64-group workload: four waves per workgroup
// (8 blocks, 64-byte line halves) beat two and eight; persistent workgroups
// that prefetch their next item were slower (the item barrier keeps the waves
// in step, and the second register set halves the waves per SIMD).
constexpr int kQuantWaves = 4;
constexpr int kQuantThreads = 64 * kQuantWaves;
constexpr int kItemBlocks = 2 * kQuantWaves;  // blocks of a work item
// bytes per staged code row: 8 per block, plus 8 to spread the LDS banks
constexpr int kStagePitch = 8 * kItemBlocks + 8;

template <int CPL>
struct Stage {
  uint8_t codes[32 * CPL * kStagePitch];
  uint8_t scales[32 * CPL * kItemBlocks];
};

// The group scales of a wave's current item and its LDS tables (recomputed
// when the item's groups change).
struct GroupTabs {
  int g0, g1;
  GScale s0, s1;
  bool fold;  // the transform's 0.25 is folded into the block maximum and the tables
};

// Folding the transform's factor 0.25: bf16(0.25 t) = 0.25 bf16(t) whenever
// 0.25 t is a normal number, so the block maximum can be taken over bf16(t)
// and scaled once, and the 0.25 can join the encode multiplier (exactly, while
// that stays normal). With the group amax in [2^-90, 2^120] the cases where
// 0.25 t is subnormal cannot change a code (such an element times any encode
// multiplier of the group stays below 2^-9, so it encodes as a signed zero
// either way, and a block made only of them gets scale code 0 either way),
// and the tables stay normal. Outside that range the unfolded path runs.
__device__ __forceinline__ bool fold_ok(float amax) { return amax >= 0x1p-90f && amax <= 0x1p120f; }

template <int CPL, bool RHT, bool SR, bool FOLD, bool FAST, int DT>
__device__ __forceinline__ void encode_columns(Tile<CPL, DT>& r, uint32_t mask, const float* tab, float enc,
                                               uint64_t blk, uint64_t nbp, uint8_t* cst, uint8_t* sst,
                                               uint64_t seed, uint32_t offset) {
  static_assert(!FOLD || FAST || DT == kInBF16, "the fold is exact only for a bf16 round-through");
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    float v16[16];
    if constexpr (RHT) column_signed<CPL, DT>(r, c, mask, v16);
    else column<CPL, DT>(r, c, v16);
    if constexpr (RHT) {
      fwht16(v16);
      if constexpr (!FAST) {
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          if constexpr (DT == kInBF16) {
            v16[i] = bf16_round(FOLD ? v16[i] : v16[i] * 0.25f);
            v16[i + 1] = bf16_round(FOLD ? v16[i + 1] : v16[i + 1] * 0.25f);
          } else {
            float a = v16[i] * 0.25f, b = v16[i + 1] * 0.25f;
            round_through2<DT>(a, b);
            v16[i] = a;
            v16[i + 1] = b;
          }
        }
      } else if constexpr (!FOLD) {
#pragma unroll
        for (int i = 0; i < 16; ++i) v16[i] *= 0.25f;
      }
    }
    float m = max16_abs(v16);
    if constexpr (FOLD) m *= 0.25f;
    const uint32_t sc = block_scale(m, enc);
    const float rc = tab[sc];
#pragma unroll
    for (int i = 0; i < 16; ++i) v16[i] = v16[i] * rc;
    uint2 out;
    if constexpr (SR) {
      const U4 wr = block_random(blk, 1, seed, offset);
      out.x = sr_pack8(v16, wr.x, wr.y);
      out.y = sr_pack8(v16 + 8, wr.z, wr.w);
    } else {
      out.x = rtne_pack8(v16);
      out.y = rtne_pack8(v16 + 8);
    }
    *reinterpret_cast<uint2*>(cst + c * kStagePitch) = out;
    sst[c * kItemBlocks] = (uint8_t)sc;
    blk += nbp;
  }
}

template <int CPL, bool RHT, bool SR, bool FAST, int DT>
__device__ __forceinline__ void encode_item(const Item& it, Tile<CPL, DT>& r, uint32_t mask, const float* gam,
                                            GroupTabs& gt, float* tabs, Stage<CPL>& st, uint32_t mpad,
                                            uint64_t seed, uint32_t offset) {
  // the 0.25 folds exactly into a bf16 round-through, or where no round-through runs
  constexpr bool kCanFold = FAST || DT == kInBF16;
  const uint32_t lane = threadIdx.x & 63, half = lane >> 5;
  const uint32_t wid = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  if (it.b0.g != gt.g0 || it.b1.g != gt.g1) {
    gt.g0 = it.b0.g;
    gt.g1 = it.b1.g;
    const float a0 = gam[gt.g0], a1 = gam[gt.g1];
    gt.s0 = global_scale(a0);
    // both blocks in one group (most pairs): one set of scales and one table
    if (gt.g1 != gt.g0) gt.s1 = global_scale(a1);
    else gt.s1 = gt.s0;
    gt.fold = kCanFold && RHT && fold_ok(a0) && fold_ok(a1);
    const float f = gt.fold ? 0.25f : 1.0f;
    // the wave's own tables: its LDS writes precede its reads
    tabs[lane] = encode_mult(lane, gt.s0.dec) * f;
    tabs[lane + 64] = encode_mult(lane + 64, gt.s0.dec) * f;
    if (gt.g1 != gt.g0) {
      tabs[128 + lane] = encode_mult(lane, gt.s1.dec) * f;
      tabs[128 + lane + 64] = encode_mult(lane + 64, gt.s1.dec) * f;
    }
  }
  const float* tab = tabs + (gt.g1 != gt.g0 ? half * 128 : 0);
  const float enc = half ? gt.s1.enc : gt.s0.enc;
  const uint64_t nbp = (uint64_t)(mpad >> 4);  // blocks per plane row
  const uint64_t blk = (uint64_t)it.col * nbp + it.tb;
  // staging slot of the lane's block: byte 8 j of code row r, byte j of
  // scale row r, j = the block's place among the item's blocks
  const uint32_t j = 2 * wid + half;
  uint8_t* cst = st.codes + (lane & 31) * CPL * kStagePitch + 8 * j;
  uint8_t* sst = st.scales + (lane & 31) * CPL * kItemBlocks + j;
  if (RHT && gt.fold)
    encode_columns<CPL, RHT, SR, kCanFold, FAST, DT>(r, mask, tab, enc, blk, nbp, cst, sst, seed, offset);
  else
    encode_columns<CPL, RHT, SR, false, FAST, DT>(r, mask, tab, enc, blk, nbp, cst, sst, seed, offset);
}

// Write-out of a staged item: plane rows of column tile ctile, blocks
// kItemBlocks bg onwards; only blocks inside the padded length (and the plane
// capacity, which only malformed offsets reach) and rows inside cols.
template <int CPL>
__device__ __forceinline__ void write_item(const Stage<CPL>& st, uint32_t ctile, uint32_t bg, uint32_t cols,
                                           uint32_t mpad, int64_t cap, uint8_t* __restrict__ codes, int64_t ldc,
                                           uint8_t* __restrict__ scales, int64_t lds) {
  constexpr int kRows = 32 * CPL;
  constexpr int kRowStep = kQuantThreads / kItemBlocks;  // plane rows between a thread's stores
  const uint32_t row0 = ctile * kRows, blkb = bg * kItemBlocks;
  const int64_t nvalid = min((int64_t)(mpad >> 4), cap >> 4) - (int64_t)blkb;  // valid blocks of the item
  // thread t: block jj = t mod 8 of plane rows t / 8 + 32 k; the byte offsets advance by whole row steps
  const uint32_t rr0 = threadIdx.x / kItemBlocks, jj = threadIdx.x % kItemBlocks;
  const bool jok = (int64_t)jj < nvalid;
  int64_t co = (int64_t)(row0 + rr0) * ldc + (int64_t)(blkb + jj) * 8;
  int64_t so = (int64_t)(row0 + rr0) * lds + blkb + jj;
  const int64_t cstep = (int64_t)kRowStep * ldc, sstep = (int64_t)kRowStep * lds;
#pragma unroll
  for (int k = 0; k < kRows / kRowStep; ++k) {
    const uint32_t rr = rr0 + k * kRowStep;
    if (jok && row0 + rr < cols) {
      *reinterpret_cast<uint2*>(codes + co) = *reinterpret_cast<const uint2*>(st.codes + rr * kStagePitch + jj * 8);
      scales[so] = st.scales[rr * kItemBlocks + jj];
    }
    co += cstep;
    so += sstep;
  }
}

// Rowwise plane from the lane's raw tile (before the transform's signs): token
// row t of the lane's block is columns col .. col + 7 of x row row_first + t,
// and with the neighbouring lane (lane ^ 1) it forms the 16-column block at
// columns col & ~15. Both lanes take the block maximum through a DPP swap and
// encode their own 8 elements (4 code bytes each; the even lane stores the
// scale). SR: for the token pair (i, i + 8) the even lane draws block i and the
// odd lane block i + 8, and each passes the other the two Philox words it needs
// (elements 0..7 of a block use words 0 and 1, elements 8..15 words 2 and 3).
template <bool SR, int DT>
__device__ __forceinline__ void encode_rows(const Tile<8, DT>& r, uint32_t col, bool ok, int row_first, int left,
                                            const float* tab, float enc, uint32_t cols,
                                            uint8_t* __restrict__ rcodes, int64_t rldc,
                                            uint8_t* __restrict__ rscales, int64_t rlds, uint64_t seed,
                                            uint32_t offset) {
  const bool odd = threadIdx.x & 1;
  const uint32_t kb = col >> 4, nbr = cols >> 4;  // the block's index in its row; blocks per row
  uint8_t* cp = rcodes + (int64_t)row_first * rldc + (col >> 1);
  uint8_t* sp = rscales + (int64_t)row_first * rlds + kb;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t wa[2], wb[2];  // words for tokens i and i + 8
    if constexpr (SR) {
      const U4 w = block_random((uint64_t)(row_first + i + (odd ? 8 : 0)) * nbr + kb, 0, seed, offset);
      const uint32_t ga = swap_pair_u(odd ? w.x : w.z), gb = swap_pair_u(odd ? w.y : w.w);
      wa[0] = odd ? ga : w.x;
      wb[0] = odd ? gb : w.y;
      wa[1] = odd ? w.z : ga;
      wb[1] = odd ? w.w : gb;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = i + 8 * h;
      float v[8];
      if constexpr (DT == kInFP32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = __uint_as_float(r[t][e]);
      } else if constexpr (DT == kInFP16) {
        widen8_h(make_uint4(r[t][0], r[t][1], r[t][2], r[t][3]), v);
      } else {
        widen8(make_uint4(r[t][0], r[t][1], r[t][2], r[t][3]), v);
      }
      float m = max8_abs(v);
      m = fmaxf(m, swap_pair(m));
      const uint32_t sc = block_scale(m, enc);
      const float rc = tab[sc];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * rc;
      uint32_t code;
      if constexpr (SR) code = sr_pack8(v, wa[h], wb[h]);
      else code = rtne_pack8(v);
      if (ok && t < left) {
        *reinterpret_cast<uint32_t*>(cp + (int64_t)t * rldc) = code;
        if (!odd) sp[(int64_t)t * rlds] = (uint8_t)sc;
      }
    }
  }
}

// Encode kernel. COL: the columnwise plane (transform if RHT), staged and
// written as described above. ROW: the rowwise plane (CPL 8: a lane pair
// holds one 16-column block of each of its 16 token rows).
template <int CPL, bool RHT, bool SR, bool FAST, bool COL, bool ROW, int DT>
__global__ __launch_bounds__(kQuantThreads) void k_grouped_quant(const void* __restrict__ x, const GroupArgs a,
                                                                 const Workspace* ws, int64_t cap, uint32_t nbg,
                                                                 uint32_t ntc, uint32_t npairs, uint32_t chunk) {
  static_assert(!ROW || CPL == 8, "the rowwise encode pairs lanes of 8 columns");
  __shared__ __align__(16) Stage<CPL> stage;
  __shared__ float rcp_tab[kQuantWaves][2][128];   // per wave: columnwise tables of its two blocks' groups
  __shared__ float rcp_row[kQuantWaves][2][128];   // per wave: rowwise tables
  const uint32_t lane = threadIdx.x & 63, half = lane >> 5;
  const uint32_t wid = (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t rows = (uint32_t)a.rows, cols = (uint32_t)a.cols;
  const uint32_t v = xcd_work_item(chunk);
  if (v >= nbg * ntc) return;  // whole workgroup
  const uint32_t ctile = v / nbg, bg = v - ctile * nbg;
  const uint32_t pair = bg * kQuantWaves + wid;
  const GroupScan q = group_scan(a.offsets, a.groups, (int)rows);
  // The first wave: padded offsets, and the groups' amax / S_dec of each plane
  // whose amax was given (otherwise the reduce kernel wrote them).
  if (v == 0 && wid == 0 && lane < (uint32_t)a.groups) {
    if (COL && a.amax_in != nullptr) {
      if (a.amax_out) a.amax_out[lane] = a.amax_in[lane];
      if (a.scale_out) a.scale_out[lane] = global_scale(a.amax_in[lane]).dec;
    }
    if (ROW && a.ramax_in != nullptr) {
      if (a.ramax_out) a.ramax_out[lane] = a.ramax_in[lane];
      if (a.rscale_out) a.rscale_out[lane] = global_scale(a.ramax_in[lane]).dec;
    }
    if (a.poff_out) a.poff_out[lane + 1] = q.ps;
    if (lane == 0 && a.poff_out) a.poff_out[0] = 0;
  }
  const uint32_t mpad = (uint32_t)lane_int(q.ps, 63);
  if (pair < npairs) {  // wave-uniform; every wave reaches the barrier below
    const Item it = item_of<CPL>(ctile, pair, q, a.groups, mpad, cols);
    Tile<CPL, DT> r;
    load_item<CPL, DT>(x, a.ld_x, (int)rows, it, true, r);
    if constexpr (ROW) {
      const float* gr = a.ramax_in ? a.ramax_in : ws->partial + kGroupAmaxRow;
      const GScale s0 = global_scale(gr[it.b0.g]), s1 = global_scale(gr[it.b1.g]);
      float* rt = &rcp_row[wid][0][0];
      rt[lane] = encode_mult(lane, s0.dec);
      rt[lane + 64] = encode_mult(lane + 64, s0.dec);
      rt[128 + lane] = encode_mult(lane, s1.dec);
      rt[128 + lane + 64] = encode_mult(lane + 64, s1.dec);
      const int t0 = (int)(it.tb * 16u) - (half ? it.b1.start : it.b0.start);
      const int row_first = (half ? it.b1.row0 : it.b0.row0) + t0;
      const int left = (half ? it.b1.n : it.b0.n) - t0;  // real tokens of the lane's block
      encode_rows<SR, DT>(r, it.col, it.ok, row_first, left, rt + half * 128, half ? s1.enc : s0.enc, cols, a.rcodes,
                      a.rldc, a.rscales, a.rlds, a.seed, a.offset);
    }
    if constexpr (COL) {
      GroupTabs gt;
      gt.g0 = -1;
      gt.g1 = -1;
      encode_item<CPL, RHT, SR, FAST, DT>(it, r, a.mask, a.amax_in ? a.amax_in : ws->partial + kGroupAmax, gt,
                                      &rcp_tab[wid][0][0], stage, mpad, a.seed, a.offset);
    }
  }
  if constexpr (COL) {
    __syncthreads();
    write_item<CPL>(stage, ctile, bg, cols, mpad, cap, a.codes, a.ldc, a.scales, a.lds);
  }
}

// Upper bound of the padded token blocks of all groups:
// sum ceil(n_g / 16) <= (rows + 15 G) / 16.
int64_t grouped_blocks(int64_t rows, int groups) { return (rows + 15 * (int64_t)groups) / 16; }

// Columns per lane: the amax pass 4 (65 registers, many waves per SIMD for
// its loads); the encode 4 for the columnwise plane alone (87 registers, five
// waves per SIMD: on the 16384 x 7168 workload the encode alone takes
// 74.0 us against 76.4 us with 8, the full step the same) and 8 when it also
// writes the rowwise plane (a lane pair's 16 columns form one rowwise block).
constexpr int kCplAmax = 4, kCplQuant = 4, kCplQuantRows = 8;

template <int CPL>
uint32_t tiles_of(int64_t cols) { return (uint32_t)((cols + 32 * CPL - 1) / (32 * CPL)); }

// Launch geometry of a pass: block pairs, block quads (one per workgroup and
// column tile), column tiles, and the XCD chunk.
struct Geo {
  uint32_t npairs, nq, ntc, chunk;
  dim3 grid;
};
template <int CPL>
Geo geo_of(int64_t cols, uint32_t nb_max) {
  Geo g;
  g.npairs = (nb_max + 1) / 2 < 1 ? 1 : (nb_max + 1) / 2;
  g.nq = (g.npairs + kWaves - 1) / kWaves;
  g.ntc = tiles_of<CPL>(cols);
  g.chunk = xcd_chunk((uint64_t)g.nq * g.ntc);
  g.grid = dim3(xcd_grid((uint64_t)g.nq * g.ntc));
  return g;
}

// Amax pass and reduce kernel for the planes whose amax is not given (COL,
// ROW); rowwise slots follow the columnwise ones when both are computed.
template <int CPLA, bool RHT, bool FAST, bool COL, bool ROW, int DT>
void launch_amax(const GroupArgs& a, uint32_t nb_max, hipStream_t s) {
  const Geo g = geo_of<CPLA>(a.cols, nb_max);
  const uint64_t items = (uint64_t)g.nq * g.ntc;
  const uint32_t nwg = (uint32_t)(items < (uint64_t)kAmaxGrid ? items : kAmaxGrid);
  const uint32_t rbase = COL ? nwg * 64 : 0;
  hipLaunchKernelGGL((k_grouped_amax<CPLA, RHT, FAST, COL, ROW, DT>), dim3(nwg), dim3(kT), 0, s, a.x, (int)a.rows,
                     (uint32_t)a.cols, a.ld_x, a.offsets, a.groups, a.mask, a.ws, g.nq, g.ntc, g.npairs, nb_max,
                     rbase);
  hipLaunchKernelGGL((k_grouped_reduce<COL, ROW>), dim3(a.groups), dim3(kReduceThreads), 0, s, a.ws, nwg, rbase,
                     a.amax_out, a.scale_out, a.ramax_out, a.rscale_out);
}

template <int CPLE, bool RHT, bool SR, bool FAST, bool COL, bool ROW, int DT>
void launch_quant(const GroupArgs& a, uint32_t nb_max, hipStream_t s) {
  const int64_t cap = COL ? (a.ldc * 2 < a.lds * 16 ? a.ldc * 2 : a.lds * 16) : 0;
  const uint32_t npairs = (nb_max + 1) / 2 < 1 ? 1 : (nb_max + 1) / 2;
  const uint32_t nbg = (npairs + kQuantWaves - 1) / kQuantWaves;  // items per column tile
  const uint32_t ntc = tiles_of<CPLE>(a.cols);
  const uint32_t chunk = xcd_chunk((uint64_t)nbg * ntc);
  hipLaunchKernelGGL((k_grouped_quant<CPLE, RHT, SR, FAST, COL, ROW, DT>), dim3(xcd_grid((uint64_t)nbg * ntc)),
                     dim3(kQuantThreads), 0, s, a.x, a, a.ws, cap, nbg, ntc, npairs, chunk);
}

template <bool RHT, bool FAST, bool COL, bool ROW, int DT>
void launch_planes(const GroupArgs& a, hipStream_t s) {
  const uint32_t nb_max = (uint32_t)grouped_blocks(a.rows, a.groups);
  const bool col_amax = COL && !a.amax_in, row_amax = ROW && !a.ramax_in;
  if (col_amax && row_amax) launch_amax<kCplAmax, RHT, FAST, true, true, DT>(a, nb_max, s);
  else if (col_amax) launch_amax<kCplAmax, RHT, FAST, true, false, DT>(a, nb_max, s);
  else if (row_amax) launch_amax<kCplAmax, false, false, false, true, DT>(a, nb_max, s);
  constexpr int kC = ROW ? kCplQuantRows : kCplQuant;
  if (a.sr) launch_quant<kC, RHT, true, FAST, COL, ROW, DT>(a, nb_max, s);
  else launch_quant<kC, RHT, false, FAST, COL, ROW, DT>(a, nb_max, s);
}

// FAST (no round-through of the transform's output) exists only with the
// transform and a columnwise plane; the rowwise plane alone has no transform.
// fp32 input has no round-through either: it always takes the FAST kernels.
template <int DT>
void launch_grouped_t(const GroupArgs& a, hipStream_t s) {
  const bool fast = a.fast || DT == kInFP32;
  if (a.col && a.row) {
    if (a.rht && fast) launch_planes<true, true, true, true, DT>(a, s);
    else if (a.rht) launch_planes<true, false, true, true, DT>(a, s);
    else launch_planes<false, false, true, true, DT>(a, s);
  } else if (a.col) {
    if (a.rht && fast) launch_planes<true, true, true, false, DT>(a, s);
    else if (a.rht) launch_planes<true, false, true, false, DT>(a, s);
    else launch_planes<false, false, true, false, DT>(a, s);
  } else {
    launch_planes<false, false, false, true, DT>(a, s);
  }
}

}  // namespace

// Workspace slots the grouped path needs: 64 per amax workgroup (at most
// kAmaxGrid) and plane, then the per-group amax of both planes; independent of
// the size of x.
int64_t grouped_partials(int64_t rows, int64_t cols, int groups, int planes) {
  (void)rows;
  (void)cols;
  (void)groups;
  return (int64_t)planes * kAmaxGrid * 64 + 128;
}

hipError_t launch_grouped(const GroupArgs& a, hipStream_t s) {
  if (a.dtype == kInFP16) launch_grouped_t<kInFP16>(a, s);
  else if (a.dtype == kInFP32) launch_grouped_t<kInFP32>(a, s);
  else launch_grouped_t<kInBF16>(a, s);
  return hipGetLastError();
}

}  // namespace nvfp4q
