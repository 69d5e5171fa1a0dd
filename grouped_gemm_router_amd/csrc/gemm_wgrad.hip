// Weight-gradient GEMMs of the MoE backward on gfx950 bf16 MFMA.  With the contraction
// running over the rows routed to expert e (LigerCute, "Backward pass": the expert-weight
// gradients; row r has token t_r and routing weight w_r):
//   dW_down[e]           = sum_r (w_r h_r)^T dY[t_r]           [I, H]
//   [dW_gate | dW_up][e] = sum_r X[t_r]^T [dg | du]_r           [H, 2I]
// The operands w h and [dg | du] are fp32 values carried as a bf16 value plus a bf16
// remainder (two parts of the operand, both contracted); dY and X are bf16 inputs, read
// straight from their token rows through row_token (no gathered copy).
//
// Both operands are "k-major": a k-tile is BK consecutive expert-major rows,
// each contiguous along M (or N).  The rows are copied to LDS unchanged by the
// direct global->LDS loads (one 16-byte chunk per lane), and the LDS transpose
// read ds_read_b64_tr_b16 turns them into MFMA operands: within each 16-lane
// group, lane i receives element i % 4 of the four-element pieces addressed by
// lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4.  Pointing lane s of a group
// at row kb + s / 4, columns c0 + 4 (s % 4) .. + 3 therefore gives lane i
// column c0 + i of rows kb .. kb + 3 -- half of the eight k values a lane of
// v_mfma_f32_32x32x16_bf16 holds.
//
// Rows past the end of an expert's segment in the last k-tile are loaded from
// the segment's last row (a valid address); the B operand's copies of them are
// then overwritten with zeros in LDS, so they add nothing.
#include "gemm_rows.h"
#include "kernels.h"

namespace moe {

// Tile configuration: BM x BN output tiles, WAVES_M x WAVES_N waves, BK-row
// k-tiles, NST LDS stages.  A stage holds the NA parts of the A k-tile and the NB
// parts of the B k-tile; MFMA pass q multiplies A part min(q, NA-1) by B part
// min(q, NB-1), all into the same accumulators.  IDS token ids of the tile's rows
// sit in LDS for a gathered operand.
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int NST_, int NA_, int NB_>
struct WgCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NW = WAVES_M_ * WAVES_N_;
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int BK = BK_, NST = NST_, NA = NA_, NB = NB_, NP = NA_ > NB_ ? NA_ : NB_;
  static constexpr int A_SLOTS = BM * BK / 8, B_SLOTS = BN * BK / 8;   // 16-byte slots per stage and part
  static constexpr int B_OFF = NA * A_SLOTS;                           // first B slot of a stage
  static constexpr int STAGE = NA * A_SLOTS + NB * B_SLOTS;
  static constexpr int EPI = STAGE * 16 / NW;                          // epilogue staging bytes per wave
  static constexpr int IDS = 2048;
  static_assert(BK % 16 == 0 && NST * STAGE * 16 + IDS * 4 <= 156 * 1024, "k-tile and LDS budget");
  static_assert(IDS % BK == 0 && IDS >= NST * BK, "whole k-tiles per id window");
};
// 32-row k-tiles and three stages (two k-tiles in flight), 48 KB each.
//   dW_down:    A = w h as bf16 value and remainder (two parts), B = dY token rows.
//   dW_gate/up: A = X token rows, B = [dg | du] as bf16 value and remainder (two parts).
using CfgWgDown = WgCfg<256, 256, 2, 4, 32, 3, 2, 1>;
using CfgWgGateUp = WgCfg<256, 256, 2, 4, 32, 3, 1, 2>;

// Loader of one k-major operand: BK rows x COLS columns (cols [c0, c0 + COLS) of
// the source rows).  Load instruction i of wave w fills LDS slots
// [64 (i NW + w), + 64): rows RPI (i NW + w) + lane / CPR.
template <class C, int COLS>
struct KMajorLoad {
  static constexpr int CPR = COLS / 8;                  // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;                  // rows per load instruction
  static constexpr int INST = C::BK * CPR / 64;
  static constexpr int PER = INST / C::NW;              // load instructions per wave and k-tile
  static_assert(CPR >= 16 && 64 % CPR == 0, "row of 128..512 bf16 columns");
  static_assert(INST % C::NW == 0 && (RPI * C::NW) % 4 == 0, "row mod 4 fixed per lane");
  uint32_t colb;                                        // byte offset of this lane's chunk in a row
  int rsub;

  // c0: first column of the tile; ncols: columns of the source (a multiple of 8).
  __device__ void init(int c0, int ncols) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rsub = lane / CPR;
    const int r = RPI * wave + rsub;                    // this lane's rows are r mod 4 for every i
    const int chunk = (lane % CPR) ^ tr_swz(r);
    colb = (uint32_t)min(c0 + chunk * 8, ncols - 8) * 2u;
  }
  // The k-tile row (before clamping) that load instruction i of this lane covers.
  __device__ int row(int i) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    return (i * C::NW + wave) * RPI + rsub;
  }
  // Load instruction i: this lane's chunk of the row at base + rowoff (bytes) into the operand's
  // LDS area at `lds`.
  __device__ void issue(const uint8_t* base, uint32_t rowoff, uint4* lds, int i) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (i * C::NW + wave) * 64;
    lds_dma16(base, rowoff + colb, lds_addr(lds + S));
  }
};

// Byte offsets (in a stage) of this lane's transpose reads for sub-step 0, read 0, part 0;
// sub-step kk, read j is at + (16 kk + 4 j) row strides; A part na at + na A_SLOTS, B part nb at
// + nb B_SLOTS.
template <class C>
struct TrFragAddr {
  static constexpr uint32_t RA = C::BM * 2, RB = C::BN * 2;       // row strides in bytes
  uint32_t a[C::FM], b[C::FN];
  __device__ void init(int wm, int wn, int lane) {
    const int s = lane & 15, g = lane >> 4;
    const int r = 8 * (g >> 1) + (s >> 2);              // k row (lanes 32-63: k + 8)
    const int sub = 2 * (g & 1) + ((s & 3) >> 1);       // chunk within the 32-column fragment
    const uint32_t in = 8u * (s & 1);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int ch = (wm * C::WTM + fm * 32) / 8 + sub;
      a[fm] = r * RA + (uint32_t)(ch ^ tr_swz(r)) * 16u + in;
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int ch = (wn * C::WTN + fn * 32) / 8 + sub;
      b[fn] = C::B_OFF * 16 + r * RB + (uint32_t)(ch ^ tr_swz(r)) * 16u + in;
    }
  }
};

// One k-tile (BK / 16 MFMA sub-steps), operand reads of sub-step kk + 1 in flight
// under the MFMAs of sub-step kk; the NLOAD load instructions of a later k-tile
// are spread over the sub-steps (as in the row-grouped GEMMs).  Every operand part
// pair accumulates into the same accumulators.
template <class C, bool LOADS, int NLOAD, class Issue>
__device__ __forceinline__ void mma_ktile_tr(const lds_u8* st, const TrFragAddr<C>& fa,
                                             f32x16 (&acc)[C::FM][C::FN], Issue issue) {
  constexpr int KK = C::BK / 16;
  constexpr int NR = 2 * (C::NA * C::FM + C::NB * C::FN), NM = C::FM * C::NP * C::FN;
  constexpr int LPS = MOE_ROWS_LPS < NLOAD ? MOE_ROWS_LPS : NLOAD;
  constexpr int LPS_ = LPS * KK >= NLOAD ? LPS : (NLOAD + KK - 1) / KK;
  static_assert(!LOADS || LPS_ * KK >= NLOAD, "every load of the k-tile must be issued");
  constexpr uint32_t RA = TrFragAddr<C>::RA, RB = TrFragAddr<C>::RB;
  bf16x8 a[2][C::NA][C::FM], b[2][C::NB][C::FN];
  auto load = [&](int kk, int buf) {
#pragma unroll
    for (int na = 0; na < C::NA; ++na)
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
        a[buf][na][fm] = tr_frag(st, fa.a[fm] + na * C::A_SLOTS * 16u + 16u * kk * RA, RA);
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        b[buf][nb][fn] = tr_frag(st, fa.b[fn] + nb * C::B_SLOTS * 16u + 16u * kk * RB, RB);
  };
  load(0, 0);
  static_for<0, KK>([&](auto kkc) {
    constexpr int kk = decltype(kkc)::value;
    constexpr int J0 = kk * LPS_, J1 = (kk + 1) * LPS_ < NLOAD ? (kk + 1) * LPS_ : NLOAD;
    constexpr int NL = LOADS && J1 > J0 ? J1 - J0 : 0;
    if constexpr (kk + 1 < KK) load(kk + 1, (kk + 1) & 1);
    static_for<0, NL>([&](auto jc) { issue(J0 + decltype(jc)::value); });
#pragma unroll
    for (int q = 0; q < C::NP; ++q)
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
          acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[kk & 1][q < C::NB ? q : C::NB - 1][fn],
                                                                a[kk & 1][q < C::NA ? q : C::NA - 1][fm],
                                                                acc[fm][fn], 0, 0, 0);
    constexpr int EARLY = kk + 1 < KK ? 2 : 0;
    if constexpr (kk + 1 < KK) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NR / 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NR - NR / 2, 0);
    }
    if constexpr (NM - EARLY > 0) __builtin_amdgcn_sched_group_barrier(0x008, NM - EARLY, 0);
    __builtin_amdgcn_sched_barrier(0);
  });
}

// Ops: M, N of dW[e]; lda / ldb in elements; A_GATHER / B_GATHER: whether the operand is read
// from token rows through row_token (one part) or from expert-major rows (a_rows(p, na) /
// b_rows(p, nb): row 0 of part na / nb; token rows: the matrix itself); epilogue.
template <class C, class Ops>
__device__ __forceinline__ void wgrad_body(const GemmArgs& p) {
  __shared__ uint4 smem[C::NST * C::STAGE];
  __shared__ int ids[C::IDS];                         // row_token of rows [wbase, wbase + IDS) of the tile
  constexpr bool GA = Ops::A_GATHER, GB = Ops::B_GATHER;
  static_assert((!GA || C::NA == 1) && (!GB || C::NB == 1), "a gathered operand has one part");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  using AL = KMajorLoad<C, C::BM>;
  using BL = KMajorLoad<C, C::BN>;
  constexpr int PERK = C::NA * AL::PER + C::NB * BL::PER;   // load instructions per k-tile per wave
  const int M = Ops::M(p), N = Ops::N(p);
  const uint32_t lda = (uint32_t)Ops::lda(p) * 2u, ldb = (uint32_t)Ops::ldb(p) * 2u;

  WeightGrad<C::BM, C::BN, C::NT> sched;
  sched.init(p.offsets, p.E, M, N);
  XcdWalk walk;
  walk.init(sched.total);
  if (!walk.valid()) return;
  TrFragAddr<C> fa;
  fa.init(wm, wn, lane);
  const lds_u8* lds = (const lds_u8*)smem;
  AL al;
  BL bl;

  // Token ids of a window of IDS rows of the tile's expert (relative rows [wbase, wbase + IDS)),
  // read by every thread; ends with a barrier.  (Plain loads: their wait also waits for the
  // direct loads in flight, once per window.)
  int ids_e = -1, wbase = 0;
  auto load_ids = [&](const Tile& t, int base_row) {
    const int n = min(C::IDS, t.k_hi - t.k_lo - base_row);
    for (int i = threadIdx.x; i < n; i += C::NT) ids[i] = p.row_token[t.k_lo + base_row + i];
    __syncthreads();
    ids_e = t.e;
    wbase = base_row;
  };

  // k-tile kt of tile t: first row (relative to the expert's), last valid row of the k-tile, and
  // for the gathered operand the byte offset of each of this lane's rows in the token matrix
  constexpr int GPER = GA ? AL::PER : GB ? BL::PER : 1;
  struct KT { int row0; int last; uint32_t goff[GPER]; };
  auto ktile = [&](const Tile& t, int kt) {
    KT r;
    r.row0 = kt * C::BK;
    r.last = min(C::BK, t.k_hi - t.k_lo - r.row0) - 1;
    if constexpr (GA || GB) {
#pragma unroll
      for (int i = 0; i < GPER; ++i) {
        const int rr = min(GA ? al.row(i) : bl.row(i), r.last);
        r.goff[i] = (uint32_t)ids[r.row0 + rr - wbase] * (GA ? lda : ldb);
      }
    }
    return r;
  };
  auto issue_one = [&](const Tile& t, const KT& k, uint4* st, int j) {
    if (j < C::NA * AL::PER) {
      const int na = j / AL::PER, i = j % AL::PER;
      uint4* dst = st + na * C::A_SLOTS;
      if constexpr (GA) {
        al.issue(reinterpret_cast<const uint8_t*>(Ops::a_rows(p, 0)), k.goff[i], dst, i);
      } else {
        const uint8_t* rows = reinterpret_cast<const uint8_t*>(Ops::a_rows(p, na)) + (size_t)(t.k_lo + k.row0) * lda;
        al.issue(rows, (uint32_t)min(al.row(i), k.last) * lda, dst, i);
      }
    } else {
      const int jb = j - C::NA * AL::PER;
      const int nb = jb / BL::PER, i = jb % BL::PER;
      uint4* dst = st + C::B_OFF + nb * C::B_SLOTS;
      if constexpr (GB) {
        bl.issue(reinterpret_cast<const uint8_t*>(Ops::b_rows(p, 0)), k.goff[i], dst, i);
      } else {
        const uint8_t* rows = reinterpret_cast<const uint8_t*>(Ops::b_rows(p, nb)) + (size_t)(t.k_lo + k.row0) * ldb;
        bl.issue(rows, (uint32_t)min(bl.row(i), k.last) * ldb, dst, i);
      }
    }
  };
  // the first NST - 1 k-tiles of tile t (with its first id window in LDS)
  auto prologue = [&](const Tile& t, int nk) {
    if constexpr (GA || GB) {
      if (t.e != ids_e || wbase != 0) load_ids(t, 0);
    }
#pragma unroll
    for (int s = 0; s < C::NST - 1; ++s)
      if (s < nk) {
        const KT k = ktile(t, s);
#pragma unroll
        for (int j = 0; j < PERK; ++j) issue_one(t, k, smem + s * C::STAGE, j);
      }
  };

  Tile tl = sched.tile(walk.t);
  int nk = (tl.k_hi - tl.k_lo + C::BK - 1) / C::BK;
  al.init(tl.m0, M);
  bl.init(tl.n0, N);
  prologue(tl, nk);
  while (true) {
    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
    // k step kt: wait for k-tile kt, then compute it while (LOADS) issuing k-tile kt + NST - 1
    auto kstep = [&](int kt, auto loads) {
      const int ahead = nk - 1 - kt;                  // k-tiles issued after this one (capped)
      // (the first step also waits for the previous tile's epilogue stores)
      if (kt == 0) wait_vmcnt<0>();
      else wait_ktiles<C::NST, PERK>(ahead < C::NST - 2 ? ahead : C::NST - 2);
      __syncthreads();
      uint4* cur = smem + (kt % C::NST) * C::STAGE;
      const int last = min(C::BK, tl.k_hi - tl.k_lo - kt * C::BK) - 1;
      if (last < C::BK - 1) {
        // rows past the segment: zeros in every B part
        const int n = (C::BK - 1 - last) * BL::CPR;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          uint4* zb = cur + C::B_OFF + nb * C::B_SLOTS + (last + 1) * BL::CPR;
          for (int i = threadIdx.x; i < n; i += C::NT) zb[i] = make_uint4(0, 0, 0, 0);
        }
        __syncthreads();
      }
      KT nx = {};
      const int nxt = kt + C::NST - 1;
      if constexpr (decltype(loads)::value) {
        // a gathered operand's next k-tile outside the id window: the next window (all waves are
        // past their reads of the current one)
        if constexpr (GA || GB) {
          if ((nxt + 1) * C::BK > wbase + C::IDS) load_ids(tl, nxt * C::BK);
        }
        nx = ktile(tl, nxt);
      }
      uint4* st = smem + (nxt % C::NST) * C::STAGE;
      auto issue = [&](int j) { issue_one(tl, nx, st, j); };
      mma_ktile_tr<C, decltype(loads)::value, PERK>(lds + (kt % C::NST) * C::STAGE * 16, fa, acc, issue);
    };
    // the last NST - 1 k steps issue nothing: peeled, not branched
    int kt = 0;
    for (; kt < nk - (C::NST - 1); ++kt) kstep(kt, std::true_type{});
    for (; kt < nk; ++kt) kstep(kt, std::false_type{});
    __syncthreads();
    const Tile done = tl;
    walk.next();
    const bool more = walk.valid();
    if (more) {
      tl = sched.tile(walk.t);
      nk = (tl.k_hi - tl.k_lo + C::BK - 1) / C::BK;
      al.init(tl.m0, M);
      bl.init(tl.n0, N);
      prologue(tl, nk);
    }
    uint8_t* wave_lds = reinterpret_cast<uint8_t*>(smem + (C::NST - 1) * C::STAGE) + wave * RowEpiLds<C>::BYTES;
    Ops::template epilogue<C>(p, done, acc, wm, wn, lane, wave_lds);
    if (!more) break;
    __syncthreads();
  }
}

// Stores the wave's 128 x 64 slab of dW[e] (rows m, columns n of a [M, ncols] matrix).
template <class C>
__device__ __forceinline__ void wg_store(uint8_t* wlds, uint16_t* out, int ld, int row0, int nrows, int col0,
                                         int ncols, f32x16 (&acc)[C::FM][C::FN], int lane) {
  stage_store_bf16<C, C::WTN, 4>(
      wlds, out, ld, row0, nrows, col0, ncols, lane,
      [&](int fm, int fn, int q, int j) { return acc[fm][fn][4 * q + j]; },
      [](int fn, int q) { return fn * 32 + q * 8; });
}

// dW_down[e] = sum_r (w_r h_r)^T dY[t_r]: A = w h rows [A, I] as bf16 values (na = 0) and bf16
// remainders (na = 1), B = dY token rows [T, H] through row_token.
struct WgDownOps {
  static constexpr bool A_GATHER = false, B_GATHER = true;
  __device__ static int M(const GemmArgs& p) { return p.I; }
  __device__ static int N(const GemmArgs& p) { return p.H; }
  __device__ static int lda(const GemmArgs& p) { return p.I; }
  __device__ static int ldb(const GemmArgs& p) { return p.H; }
  __device__ static const uint16_t* a_rows(const GemmArgs& p, int na) { return na ? p.hw_lo : p.hw; }
  __device__ static const uint16_t* b_rows(const GemmArgs& p, int) { return p.dY; }
  template <class C>
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                                  int lane, uint8_t* wlds) {
    wg_store<C>(wlds, p.dWd + (size_t)t.e * p.I * p.H, p.H, t.m0 + wm * C::WTM, p.I, t.n0 + wn * C::WTN, p.H, acc,
                lane);
  }
};

// [dW_gate | dW_up][e] = sum_r X[t_r]^T [dg | du]_r: A = X token rows [T, H] through row_token,
// B = [dg | du] rows [A, 2I] as bf16 values (nb = 0) and bf16 remainders (nb = 1).
// The ungated (ReLU^2) expert has du rows [A, I] only and gets dW_up alone.
struct WgGateUpOps {
  static constexpr bool A_GATHER = true, B_GATHER = false;
  __device__ static int M(const GemmArgs& p) { return p.H; }
  __device__ static int N(const GemmArgs& p) { return act_gated(p.act) ? 2 * p.I : p.I; }
  __device__ static int lda(const GemmArgs& p) { return p.H; }
  __device__ static int ldb(const GemmArgs& p) { return N(p); }
  __device__ static const uint16_t* a_rows(const GemmArgs& p, int) { return p.X; }
  __device__ static const uint16_t* b_rows(const GemmArgs& p, int nb) { return nb ? p.dGU_lo : p.dGU; }
  template <class C>
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                                  int lane, uint8_t* wlds) {
    // I is a multiple of 64, so a wave's 64 columns are all gate or all up
    const int col0 = t.n0 + wn * C::WTN;
    // (ungated: every column is an up column, and columns past I are not stored)
    const bool gated = act_gated(p.act);
    const bool up = !gated || col0 >= p.I;
    uint16_t* out = (up ? p.dWu : p.dWg) + (size_t)t.e * p.H * p.I;
    wg_store<C>(wlds, out, p.I, t.m0 + wm * C::WTM, p.H, gated && up ? col0 - p.I : col0, p.I, acc, lane);
  }
};

__global__ void __launch_bounds__(CfgWgDown::NT) k_bwd_dw_down(const GemmArgs p) {
  wgrad_body<CfgWgDown, WgDownOps>(p);
}
__global__ void __launch_bounds__(CfgWgGateUp::NT) k_bwd_dw_gateup(const GemmArgs p) {
  wgrad_body<CfgWgGateUp, WgGateUpOps>(p);
}

template <class C>
static int wgrad_grid(const GemmArgs& a, int M, int N) {
  long tiles = (long)a.E * ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  long cap = (long)num_cus();            // one workgroup per CU (LDS)
  long g = tiles < cap ? tiles : cap;
  return (int)((g + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
}

hipError_t launch_bwd_dw_down(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_dw_down, dim3(wgrad_grid<CfgWgDown>(a, a.I, a.H)), dim3(CfgWgDown::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bwd_dw_gateup(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_dw_gateup, dim3(wgrad_grid<CfgWgGateUp>(a, a.H, act_gated(a.act) ? 2 * a.I : a.I)),
                     dim3(CfgWgGateUp::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
