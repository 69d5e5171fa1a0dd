// Tile schedules of the persistent grouped GEMMs on gfx950 MFMA (the loaders
// and k loops live in gemm_rows.h and gemm_wgrad.hip).
//
// Two schedules:
//  * RowGroups: M is the ragged run of rows of each expert (expert_offsets).
//    Only experts with rows get tiles, so an unused expert's weights are never
//    read.
//  * WeightGrad: one fixed M x N output per expert; the contraction runs over
//    the expert's rows.  Experts without rows produce zero tiles.
//
// Tiles are handed out persistently: the block of id b runs on XCD b % 8 and
// takes a contiguous share of the tile list (expert-major, N fastest), so the
// blocks of one XCD work on the same expert's weights and rows and share that
// XCD's L2.
#pragma once

#include "common.h"

namespace moe {

constexpr int NUM_XCD = 8;

struct Tile {
  int e;       // expert
  int m0;      // first output row (RowGroups: absolute expert-major row)
  int m_end;   // RowGroups: end of the expert's rows; WeightGrad: M
  int n0;      // first output column
  int k_lo;    // WeightGrad: first row of the expert; RowGroups: 0
  int k_hi;    // WeightGrad: end of the expert's rows; RowGroups: K
  int nt;      // index of the N tile
};

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of up to 4 * NT values held 4 per thread.
// ---------------------------------------------------------------------------
// The lane index passes through an empty asm and the shifts are explicit ds_bpermute reads: the
// source addresses are computed here, not shared with another scan of the same kernel and held in
// registers in between.
template <int NT>
__device__ int block_exclusive_scan(int v, int* red /* NT/64 + 1 ints */) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    // lanes below d read a wrapped lane (bits 7:2 of the address) and keep their own value
    const int y = __builtin_amdgcn_ds_bpermute((lane - d) << 2, x);
    if (lane >= d) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int w = 0; w < NT / 64; ++w) {
      int t = red[w];
      red[w] = acc;
      acc += t;
    }
    red[NT / 64] = acc;
  }
  __syncthreads();
  return red[wave] + x - v;
}

// ---------------------------------------------------------------------------
// Schedules
// ---------------------------------------------------------------------------
// Which rows of each expert a RowGroups schedule covers (n rows = q * BMF + r, r < BMF):
//   ROWS_ALL:    all n rows in tiles of BM;
//   ROWS_FULL:   the q full blocks of BMF = BM rows, plus the remainder when r > 3 BMF / 4 (one
//                partly filled tile);
//   ROWS_REM_Q3: the remainder when BMF / 2 < r <= 3 BMF / 4, in one tile of BM = 3 BMF / 4 rows;
//   ROWS_REM_Q2: the remainder when BMF / 4 < r <= BMF / 2, in one tile of BM = BMF / 2 rows;
//   ROWS_REM_Q1: the remainder when 0 < r <= BMF / 4, in one tile of BM = BMF / 4 rows.
// FULL and the three REM schedules with the same BMF cover every row exactly once, and
// every expert's remainder is one tile at most BMF / 4 - 1 rows taller than it.
enum RowPart { ROWS_ALL = 0, ROWS_FULL = 1, ROWS_REM_Q1 = 2, ROWS_REM_Q2 = 3, ROWS_REM_Q3 = 4 };

template <int BM, int BN, int NT, int PART = ROWS_ALL, int BMF = BM, int GROUP_M = 1>
struct RowGroups {
  static constexpr int QUARTER = PART >= ROWS_REM_Q1 ? PART - ROWS_REM_Q1 + 1 : 0;
  static_assert(PART != ROWS_FULL || BMF == BM, "full tiles are BMF rows");
  static_assert(QUARTER == 0 || (BMF % 4 == 0 && BM * 4 == QUARTER * BMF), "one remainder tile per class");
  static constexpr int MAX_E = 1024;
  static_assert(GROUP_M >= 1, "m-tiles per group");
  // tiles of expert e with n rows, and the first of its rows they cover
  __device__ static int count(int n) {
    if constexpr (PART == ROWS_ALL) return (n + BM - 1) / BM;
    const int q = n / BMF, r = n - q * BMF;
    if constexpr (PART == ROWS_FULL) return q + (r > 3 * BMF / 4 ? 1 : 0);
    return (r > (QUARTER - 1) * BMF / 4 && r <= QUARTER * BMF / 4) ? 1 : 0;
  }
  __device__ static int first_row(int n) { return QUARTER ? n / BMF * BMF : 0; }
  int* prefix;   // LDS [E+1]: exclusive prefix of per-expert m-tile counts
  int E, ntiles_n, total, K;
  const int32_t* offsets;

  __device__ void init(const int32_t* offs, int E_, int N, int K_, int* lds_prefix, int* red) {
    prefix = lds_prefix;
    E = E_;
    K = K_;
    offsets = offs;
    ntiles_n = (N + BN - 1) / BN;
    // each thread owns 4 consecutive experts (the thread index passes through an empty asm: the
    // addresses derived from it are computed here, not shared with another schedule of the same
    // kernel and held in registers through the passes in between)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    int cnt[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid * 4 + i;
      cnt[i] = (e < E) ? count(offs[e + 1] - offs[e]) : 0;
      sum += cnt[i];
    }
    int ex = block_exclusive_scan<NT>(sum, red);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = tid * 4 + i;
      if (e < E) prefix[e] = ex;
      ex += cnt[i];
    }
    if (threadIdx.x == 0) prefix[E] = red[NT / 64];
    __syncthreads();
    total = prefix[E] * ntiles_n;
  }

  // Tile t of the schedule.  An expert's tiles are contiguous.  With GROUP_M = 1 they run m-tile
  // by m-tile, n fastest.  Otherwise they run in groups of GROUP_M m-tiles, n-tiles outermost
  // inside a group: the workgroups of one XCD that run at the same time (consecutive tiles) then
  // share GROUP_M row blocks and a few weight column blocks, and the next n-tiles of the group
  // find the row blocks still in L2; this pays where the K extent is short (row blocks of a few
  // hundred KB) and N is wide.
  // Tile t's fields (expert, first row, end of the expert's rows, first column) in v[0..3]; each
  // lane may look up a different tile.
  __device__ void tile_lane(int t, int (&v)[4]) const {
    const int mt_lin = t / ntiles_n;
    // largest e with prefix[e] <= mt_lin (experts with no tiles have prefix[e] == prefix[e+1])
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= mt_lin) lo = mid; else hi = mid - 1;
    }
    const int li = t - prefix[lo] * ntiles_n;            // tile index inside the expert
    const int me = prefix[lo + 1] - prefix[lo];           // its m-tiles
    int mt, nt;
    if constexpr (GROUP_M == 1) {
      mt = li / ntiles_n;
      nt = li - mt * ntiles_n;
    } else {
      const int g = li / (GROUP_M * ntiles_n), r = li - g * GROUP_M * ntiles_n;
      const int gm = min(GROUP_M, me - g * GROUP_M);      // m-tiles in this group
      mt = g * GROUP_M + r % gm;
      nt = r / gm;
    }
    const int o0 = offsets[lo], o1 = offsets[lo + 1];
    v[0] = lo;
    v[1] = o0 + first_row(o1 - o0) + mt * BM;
    v[2] = o1;
    v[3] = nt * BN;
  }
  // the tile of wave-uniform fields v, in scalar registers
  __device__ Tile tile_of(const int (&v)[4]) const {
    Tile tl;
    tl.e = __builtin_amdgcn_readfirstlane(v[0]);
    tl.m0 = __builtin_amdgcn_readfirstlane(v[1]);
    tl.m_end = __builtin_amdgcn_readfirstlane(v[2]);
    tl.n0 = __builtin_amdgcn_readfirstlane(v[3]);
    tl.nt = tl.n0 / BN;
    tl.k_lo = 0;
    tl.k_hi = K;
    return tl;
  }
  // every lane computes the same tile
  __device__ Tile tile(int t) const {
    int v[4];
    tile_lane(t, v);
    return tile_of(v);
  }
};

// This workgroup's tiles of an XcdWalk, one per lane: lane j looks up the fields of the
// workgroup's tile j once, when a pass starts (the schedule's LDS may be reused afterwards), and
// get(i) reads them back with v_readlane.  Launches size their grids so that no workgroup gets
// more than 64 tiles of one pass (lanes_grid).
constexpr int LANE_TILES = 64;
template <class S>
struct LaneTiles {
  int n;                   // this workgroup's tiles, at most LANE_TILES
  int v[4];                // lane j: the fields of tile j
  __device__ void init(const S& s, int t0, int step, int end) {
    n = t0 < end ? (end - t0 + step - 1) / step : 0;
    if (n > 0) {
      const int t = t0 + (int)(threadIdx.x & 63) * step;
      s.tile_lane(t < end ? t : t0, v);                 // lanes past the last tile repeat the first
    }
  }
  __device__ Tile get(const S& s, int i) const {
    int u[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) u[f] = __builtin_amdgcn_readlane(v[f], i);
    return s.tile_of(u);
  }
};

// Grid of a persistent launch over at most `tiles_bound` tiles per pass: one workgroup per CU
// (`cap`, rounded to the XCD count), or, when XcdWalk would then deal a workgroup more than
// LANE_TILES tiles of a pass, the next multiple of that grid that deals at most LANE_TILES (the
// extra workgroups run in whole rounds after the first, each with an equal share).
inline int lanes_grid(long tiles_bound, long cap) {
  long c = (cap + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
  if (tiles_bound < c) c = (tiles_bound + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
  if (c < NUM_XCD) c = NUM_XCD;
  const long per_xcd = (tiles_bound + NUM_XCD - 1) / NUM_XCD;    // tiles of the busiest XCD
  const long bpx = (per_xcd + LANE_TILES - 1) / LANE_TILES;       // workgroups per XCD it needs
  const long g = bpx * NUM_XCD;
  return (int)(g > c ? (g + c - 1) / c * c : c);
}

template <int BM, int BN, int NT>
struct WeightGrad {
  int E, M, ntiles_m, ntiles_n, total;
  const int32_t* offsets;

  __device__ void init(const int32_t* offs, int E_, int M_, int N) {
    offsets = offs;
    E = E_;
    M = M_;
    ntiles_m = (M + BM - 1) / BM;
    ntiles_n = (N + BN - 1) / BN;
    total = E * ntiles_m * ntiles_n;
  }

  __device__ Tile tile(int t) const {
    int per_e = ntiles_m * ntiles_n;
    int e = t / per_e;
    int r = t - e * per_e;
    int mt = r / ntiles_n, nt = r - mt * ntiles_n;
    Tile tl;
    tl.e = e;
    tl.m0 = mt * BM;
    tl.m_end = M;
    tl.n0 = nt * BN;
    tl.nt = nt;
    tl.k_lo = offsets[e];
    tl.k_hi = offsets[e + 1];
    return tl;
  }
};

// XCD-aware persistent walk: XCD x owns tiles [x*tpx, (x+1)*tpx), dealt round-robin to its
// bpx workgroups.  For several schedules run one after another by the same grid, `carry`
// continues the deal where the previous schedule stopped on this XCD, so that the
// workgroups that took one tile more in one schedule are not also first in the next; init
// returns the carry for the following schedule (0 starts a fresh deal).
struct XcdWalk {
  int t, step, end;
  __device__ int init(int total, int carry = 0) {
    const int G = gridDim.x;            // a multiple of NUM_XCD
    const int xcd = blockIdx.x % NUM_XCD;
    const int local = blockIdx.x / NUM_XCD;
    const int bpx = G / NUM_XCD;
    const int tpx = (total + NUM_XCD - 1) / NUM_XCD;
    int first = local - carry;
    if (first < 0) first += bpx;
    t = xcd * tpx + first;
    step = bpx;
    end = min(total, (xcd + 1) * tpx);
    const int here = max(0, end - xcd * tpx);
    return (carry + here) % bpx;
  }
  __device__ bool valid() const { return t < end; }
  __device__ void next() { t += step; }
};

// Output coordinates of accumulator element v of fragment (fm, fn) inside the
// block tile.  The MFMA is issued as (B, A), i.e. it computes the transposed
// 32x32 product, so a lane owns one output row (lane % 32) and, for each group
// q = v / 4, four consecutive columns 8q + 4 * (lane / 32) + (v % 4).
template <class C>
struct Frag {
  __device__ static int row(int wm, int fm, int lane) { return wm * C::WTM + fm * 32 + (lane & 31); }
  __device__ static int col(int wn, int fn, int q, int lane) {
    return wn * C::WTN + fn * 32 + q * 8 + (lane >> 5) * 4;
  }
};

}  // namespace moe
