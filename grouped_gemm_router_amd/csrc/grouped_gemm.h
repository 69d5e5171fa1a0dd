// Persistent grouped GEMM on gfx950 bf16 MFMA (v_mfma_f32_32x32x16_bf16).
//
// One template serves every expert GEMM of the layer.  A block owns a BM x BN
// output tile; the k loop streams 64-wide k-tiles of both operands through a
// two-stage LDS ring.  In LDS both operands are stored "K-contiguous": one
// 128-byte row per output row / column, 8 chunks of 16 bytes permuted per row
// (lds_chunk) so the 32-row MFMA operand reads are free of bank conflicts.
//
// Two ways to fill a tile:
//  * KRows loaders read rows whose contraction axis is contiguous in memory
//    (gathered token rows, expert-major activation rows, packed [E, N, K]
//    weights) with one 16-byte load per chunk.
//  * MNRows loaders read a k-tile whose rows are the contraction index (the
//    token rows of a weight-gradient GEMM, contiguous along M or N); every
//    thread loads an 8x8 block and transposes it in registers.
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

constexpr int BK = 64;
constexpr int NUM_XCD = 8;

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M * WAVES_N;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int LDS_A = BM * 8, LDS_B = BN * 8;      // uint4 units per stage
  static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B) * 16;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
};

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
template <int NT>
__device__ int block_exclusive_scan(int v, int* red /* NT/64 + 1 ints */) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
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
template <int BM, int BN, int NT>
struct RowGroups {
  static constexpr int MAX_E = 1024;
  int* prefix;   // LDS [E+1]: exclusive prefix of per-expert m-tile counts
  int E, ntiles_n, total, K;
  const int32_t* offsets;

  __device__ void init(const int32_t* offs, int E_, int N, int K_, int* lds_prefix, int* red) {
    prefix = lds_prefix;
    E = E_;
    K = K_;
    offsets = offs;
    ntiles_n = (N + BN - 1) / BN;
    // each thread owns 4 consecutive experts
    int cnt[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = threadIdx.x * 4 + i;
      cnt[i] = (e < E) ? (offs[e + 1] - offs[e] + BM - 1) / BM : 0;
      sum += cnt[i];
    }
    int ex = block_exclusive_scan<NT>(sum, red);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int e = threadIdx.x * 4 + i;
      if (e < E) prefix[e] = ex;
      ex += cnt[i];
    }
    if (threadIdx.x == 0) prefix[E] = red[NT / 64];
    __syncthreads();
    total = prefix[E] * ntiles_n;
  }

  __device__ Tile tile(int t) const {
    int mt = t / ntiles_n, nt = t - mt * ntiles_n;
    // largest e with prefix[e] <= mt (experts with no tiles have prefix[e] == prefix[e+1])
    int lo = 0, hi = E - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (prefix[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    // every lane computes the same tile: keep its fields in scalar registers
    Tile tl;
    tl.e = __builtin_amdgcn_readfirstlane(lo);
    tl.m0 = __builtin_amdgcn_readfirstlane(offsets[lo] + (mt - prefix[lo]) * BM);
    tl.m_end = __builtin_amdgcn_readfirstlane(offsets[lo + 1]);
    tl.n0 = __builtin_amdgcn_readfirstlane(nt * BN);
    tl.nt = __builtin_amdgcn_readfirstlane(nt);
    tl.k_lo = 0;
    tl.k_hi = K;
    return tl;
  }
};

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

// XCD-aware persistent walk: XCD x owns tiles [x*tpx, (x+1)*tpx).
struct XcdWalk {
  int t, step, end;
  __device__ void init(int total) {
    const int G = gridDim.x;            // a multiple of NUM_XCD
    const int xcd = blockIdx.x % NUM_XCD;
    const int local = blockIdx.x / NUM_XCD;
    const int bpx = G / NUM_XCD;
    const int tpx = (total + NUM_XCD - 1) / NUM_XCD;
    t = xcd * tpx + local;
    step = bpx;
    end = min(total, (xcd + 1) * tpx);
  }
  __device__ bool valid() const { return t < end; }
  __device__ void next() { t += step; }
};

// ---------------------------------------------------------------------------
// Loaders: K-contiguous rows
// ---------------------------------------------------------------------------
// Src must provide: __device__ static const uint16_t* rows(const P&, const Tile&, int row): the
// address of element k = 0 of a tile row, or null for a row of zeros; static int ksplit(const P&)
// and static long delta(const P&): columns k >= ksplit are read at row + delta + (k - ksplit)
// (a second matrix appended along the contraction axis; ksplit >= K when there is none).
template <int ROWS, int NT, class Src, class P>
struct KRows {
  static constexpr int CHUNKS = ROWS * 8;
  static constexpr int PER = (CHUNKS + NT - 1) / NT;
  const uint16_t* ptr[PER];
  uint4 reg[PER];
  int ksplit;
  long delta;

  __device__ void init(const P& p, const Tile& tl) {
    ksplit = Src::ksplit(p);
    delta = Src::delta(p);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      ptr[i] = nullptr;
      if (c < CHUNKS) {
        const uint16_t* q = Src::rows(p, tl, c >> 3);
        ptr[i] = q ? q + (c & 7) * 8 : nullptr;
      }
    }
  }
  __device__ void load(int k0, int /*phase*/) {
    const long off = (k0 < ksplit) ? (long)k0 : delta + (k0 - ksplit);
#pragma unroll
    for (int i = 0; i < PER; ++i)
      reg[i] = ptr[i] ? *reinterpret_cast<const uint4*>(ptr[i] + off) : make_uint4(0, 0, 0, 0);
  }
  __device__ void store(uint4* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int c = threadIdx.x + i * NT;
      if (c < CHUNKS) lds[lds_chunk(c >> 3, c & 7)] = reg[i];
    }
  }
};

// ---------------------------------------------------------------------------
// Loaders: rows are the contraction index (weight-gradient operands)
// ---------------------------------------------------------------------------
// Src must provide: __device__ const uint16_t* row(const P&, const Tile&, int r, int phase) for an
// absolute expert-major row r in [k_lo, k_hi), pointing at element 0 of the MN axis (phase: which
// pass over the rows, see Ops::PHASES); float scale(const P&, int r) and static constexpr bool SCALED.
template <int COLS, int NT, class Src, class P>
struct MNRows {
  static constexpr int BLOCKS = COLS;            // 8 (k) x COLS/8 (mn) blocks of 8x8
  static constexpr int PER = (BLOCKS + NT - 1) / NT;
  uint4 reg[PER][8];
  float scl[PER][8];
  int mn_off[PER];
  int mn_lim;
  const P* pp;
  Tile tl;

  __device__ void init(const P& p, const Tile& t, int mn0, int mn_total) {
    pp = &p;
    tl = t;
    mn_lim = mn_total;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int b = threadIdx.x + i * NT;
      int mb = b % (COLS / 8);
      mn_off[i] = mn0 + mb * 8;
    }
  }
  __device__ void load(int k0, int phase) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int b = threadIdx.x + i * NT;
      int kb = b / (COLS / 8);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        int r = tl.k_lo + k0 + kb * 8 + j;
        bool ok = (b < BLOCKS) && (r < tl.k_hi) && (mn_off[i] < mn_lim);
        if (ok) {
          reg[i][j] = *reinterpret_cast<const uint4*>(Src::row(*pp, tl, r, phase) + mn_off[i]);
          if constexpr (Src::SCALED) scl[i][j] = Src::scale(*pp, r);
        } else {
          reg[i][j] = make_uint4(0, 0, 0, 0);
          if constexpr (Src::SCALED) scl[i][j] = 0.f;
        }
      }
    }
  }
  __device__ static uint32_t half(const uint4& v, int idx) {
    uint32_t w = (idx < 2) ? ((idx == 0) ? v.x : v.y) : ((idx == 2) ? v.z : v.w);
    return w;
  }
  __device__ void store(uint4* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int b = threadIdx.x + i * NT;
      if (b >= BLOCKS) continue;
      int kb = b / (COLS / 8), mb = b % (COLS / 8);
      uint32_t w[8][4];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        w[j][0] = reg[i][j].x; w[j][1] = reg[i][j].y; w[j][2] = reg[i][j].z; w[j][3] = reg[i][j].w;
        if constexpr (Src::SCALED) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float lo = bf16_to_f32(w[j][q] & 0xffffu) * scl[i][j];
            float hi = bf16_to_f32(w[j][q] >> 16) * scl[i][j];
            w[j][q] = pack_bf16x2(lo, hi);
          }
        }
      }
#pragma unroll
      for (int mm = 0; mm < 8; ++mm) {
        const int q = mm >> 1;
        const bool odd = mm & 1;
        uint4 o;
        uint32_t d[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          uint32_t a = w[2 * jj][q], c = w[2 * jj + 1][q];
          d[jj] = odd ? ((a >> 16) | (c & 0xffff0000u)) : ((a & 0xffffu) | (c << 16));
        }
        o.x = d[0]; o.y = d[1]; o.z = d[2]; o.w = d[3];
        lds[lds_chunk(mb * 8 + mm, kb)] = o;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// MFMA over one k-tile held in LDS
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void mma_ktile(const uint4* As, const uint4* Bs, f32x16 (&acc)[C::FM][C::FN],
                                          int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    bf16x8 a[C::FM], b[C::FN];
    const int ch = kk * 2 + (lane >> 5);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      uint4 v = As[lds_chunk(wm * C::WTM + fm * 32 + (lane & 31), ch)];
      a[fm] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      uint4 v = Bs[lds_chunk(wn * C::WTN + fn * 32 + (lane & 31), ch)];
      b[fn] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[fn], a[fm], acc[fm][fn], 0, 0, 0);
  }
}

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

// ---------------------------------------------------------------------------
// The kernel body shared by every variant.  Sched is RowGroups or WeightGrad;
// Ops supplies the loaders and the epilogue for one GEMM of the layer.
// ---------------------------------------------------------------------------
template <class C, class Ops, class P>
__device__ __forceinline__ void grouped_gemm_body(const P& p) {
  __shared__ uint4 smem[2 * (C::LDS_A + C::LDS_B)];
  __shared__ int sched_lds[1024 + 1 + C::NT / 64 + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;

  typename Ops::Sched sched;
  Ops::init_sched(sched, p, sched_lds, sched_lds + 1025);
  XcdWalk walk;
  walk.init(sched.total);
  for (; walk.valid(); walk.next()) {
    const Tile tl = sched.tile(walk.t);
    typename Ops::ALoad al;
    typename Ops::BLoad bl;
    Ops::init_loaders(al, bl, p, tl);
    // Ops::PHASES passes over the contraction range (the second pass of a
    // two-phase GEMM adds the low-order bf16 part of one operand)
    const int nk1 = (tl.k_hi - tl.k_lo + BK - 1) / BK;
    const int nk = nk1 * Ops::PHASES;

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;

    if (nk > 0) {
      uint4* const As = smem;                       // stage s at As + s * LDS_A
      uint4* const Bs = smem + 2 * C::LDS_A;        // stage s at Bs + s * LDS_B
      al.load(0, 0);
      bl.load(0, 0);
      al.store(As);
      bl.store(Bs);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
          const int ph = (kt + 1) / nk1;
          const int k0 = (kt + 1 - ph * nk1) * BK;
          al.load(k0, ph);
          bl.load(k0, ph);
        }
        mma_ktile<C>(As + cur * C::LDS_A, Bs + cur * C::LDS_B, acc, wm, wn, lane);
        if (kt + 1 < nk) {
          al.store(As + (cur ^ 1) * C::LDS_A);
          bl.store(Bs + (cur ^ 1) * C::LDS_B);
        }
        __syncthreads();
      }
    }
    Ops::epilogue(p, tl, acc, wm, wn, lane);
  }
}

}  // namespace moe
