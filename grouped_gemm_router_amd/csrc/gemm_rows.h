// Grouped GEMM over ragged expert row groups, fed by gfx950's direct
// global->LDS loads (global_load_lds_dwordx4).
//
// Each wave-level load instruction writes 64 consecutive 16-byte LDS slots
// (lane l -> slot l).  The LDS tile keeps the K-contiguous, chunk-permuted
// layout the MFMA operand reads want (one row of BK bf16 = CPR chunks of 16
// bytes, chunk c of row r stored at position c ^ f(r)); the permutation is
// applied on the global side instead: the lane that owns LDS slot s loads
// chunk (s % CPR) ^ f(row) of row s / CPR.  Eight (CPR = 8) or four (CPR = 4)
// consecutive lanes still read one contiguous 128 / 64-byte piece of a row.
//
// No staging registers: NST stages of the k loop are in flight in LDS, so the
// latency of NST-1 k-tiles is hidden behind the MFMAs.  Rows past the end of
// an expert's segment (or columns past N) are loaded from a valid clamped row
// and never stored, so every load is unconditional.
#pragma once

#include <type_traits>

#include "grouped_gemm.h"

#ifndef MOE_ROWS_LPS
#define MOE_ROWS_LPS 4
#endif

namespace moe {

// Calls f(std::integral_constant<int, i>) for i in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// EPI_: bytes of LDS scratch per wave for the epilogue's staging (default: a stage's share).
template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int NST_, int EPI_ = 0>
struct RowCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NW = WAVES_M_ * WAVES_N_;
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int BK = BK_, CPR = BK_ / 8, NST = NST_;
  static constexpr int A_SLOTS = BM * CPR, B_SLOTS = BN * CPR;      // 16-byte slots per stage
  static constexpr int STAGE = A_SLOTS + B_SLOTS;
  static constexpr int EPI = EPI_ ? EPI_ : STAGE * 16 / NW;
  static_assert(CPR == 4 || CPR == 8, "k-tile of 32 or 64 bf16");
  static_assert(A_SLOTS % (64 * NW) == 0 && B_SLOTS % (64 * NW) == 0, "whole load instructions per wave");
};

// Chunk position of chunk c in row r (CPR chunks per row).  Conflict-free for
// the 32 rows of one MFMA operand read, for 8- and 16-lane LDS phases.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 8) return (r ^ (r >> 3)) & 7;
  else return ((r >> 1) ^ (r >> 3)) & 3;
}

// k-major operand tiles (rows along the contraction axis, contiguous along M or N) and
// their MFMA operand reads.  ds_read_b64_tr_b16: within each 16-lane group, lane i receives
// element i % 4 of the four-element pieces addressed by lanes i / 4, 4 + i / 4, 8 + i / 4 and
// 12 + i / 4.  Pointing lane s of a group at row kb + s / 4, columns c0 + 4 (s % 4) .. + 3
// therefore gives lane i column c0 + i of rows kb .. kb + 3 -- half of the eight k values a
// lane of v_mfma_f32_32x32x16_bf16 holds (tr_frag reads both halves).
typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4nt __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2nt __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Chunk position in a k-major LDS row: chunk c of row r sits at c ^ tr_swz(r).
// The flip of chunk-index bits 1-3 by r mod 4 makes the four rows one transpose
// read touches land in different banks, for both 16- and 32-lane LDS phases.
__device__ __forceinline__ int tr_swz(int r) { return ((r & 1) ? 10 : 0) ^ ((r & 2) ? 4 : 0); }

// Eight k values of one operand lane from a k-major tile: rows off and off + 4 row strides.
__device__ __forceinline__ bf16x8 tr_frag(const lds_u8* st, uint32_t off, uint32_t rs) {
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(st + off));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(st + off + 4 * rs));
  const v8s v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Byte offset, inside a k-major tile of `cols` columns (row stride 2 cols bytes), of this
// lane's transpose read for the 32 columns starting at col0, sub-step 0 (sub-step kk: + 16 kk
// row strides).
__device__ __forceinline__ uint32_t tr_offset(int col0, int cols, int lane) {
  const int s = lane & 15, g = lane >> 4;
  const int r = 8 * (g >> 1) + (s >> 2);              // k row (lanes 32-63: k + 8)
  const int sub = 2 * (g & 1) + ((s & 3) >> 1);       // chunk within the 32-column fragment
  const int ch = col0 / 8 + sub;
  return (uint32_t)r * (uint32_t)(cols * 2) + (uint32_t)(ch ^ tr_swz(r)) * 16u + 8u * (s & 1);
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One direct global->LDS load: 64 lanes x 16 bytes from base + voff (per lane) to
// LDS [lds, lds + 1024) (lane l at lds + 16 l).  Written as inline assembly so that
// the compiler's wait insertion, which cannot tell the LDS range it writes from
// the stage being read, does not make every later LDS read wait for it; the
// loops wait for these loads explicitly (s_waitcnt vmcnt) before the barrier
// that publishes a stage.
// A wave-uniform pointer as a scalar-register value (the compiler may compute one in vector
// registers, which an "s" operand of inline assembly cannot take).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ void lds_dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(base)), "s"(lds)
               : "m0");
}

// The lane index as a value the compiler cannot see through: addresses derived
// from it are computed where they are used instead of being hoisted out of the
// tile loop and held in registers (or spilled) across the k loop.
__device__ __forceinline__ int opaque_lane(int lane) {
  asm volatile("" : "+v"(lane));
  return lane;
}

// Loader of one operand: rows [0, ROWS) of the tile.  Src provides
//   static const uint16_t* base(const P&, const Tile&, int row0, int k0): wave-uniform base of the
//       rows [row0, row0 + 64 / CPR) for k-tile k0 (element 0 of the k-tile);
//   static uint32_t row_off(const P&, const Tile&, int row): element offset of the (clamped, valid)
//       row relative to that base.
// OPAQUE recomputes the lane-derived part of the offsets at every tile instead of letting the
// compiler hold it across the tile loop (for kernels short of registers; it costs VALU work at
// each tile start).
template <class C, int ROWS, class Src, class P, bool OPAQUE = false>
struct DirectRows {
  static constexpr int INST = ROWS * C::CPR / 64;        // load instructions per stage
  static constexpr int PER = INST / C::NW;               // ... per wave
  uint32_t off[PER];                                     // byte offsets from the wave-uniform base

  __device__ void init(const P& p, const Tile& tl) {
    const int lane = OPAQUE ? opaque_lane(threadIdx.x & 63) : (threadIdx.x & 63), wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int s = (i * C::NW + wave) * 64 + lane;
      const int row = s / C::CPR;
      const int chunk = (s % C::CPR) ^ swz<C::CPR>(row);
      off[i] = (Src::row_off(p, tl, row) + chunk * 8) * 2u;
    }
  }
  // Issue load instruction i (< PER) of k-tile k0 into the stage at `lds` (uint4 slots):
  // scalar base + 32-bit vector offset.
  __device__ void issue_one(const P& p, const Tile& tl, int k0, uint4* lds, int i) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (i * C::NW + wave) * 64;
    const uint8_t* b = reinterpret_cast<const uint8_t*>(Src::base(p, tl, S / C::CPR, k0));
    lds_dma16(b, off[i], lds_addr(lds + S));
  }
  // Issue the loads of k-tile k0 into the stage at `lds` (uint4 slots).
  __device__ void issue(const P& p, const Tile& tl, int k0, uint4* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) issue_one(p, tl, k0, lds, i);
  }
};

// Loader of a k-major B operand of the row-grouped GEMMs: the BK x BN k-tile of a [K, N]
// matrix whose k-rows are contiguous along N (the packed weights read transposed).  Src
// provides kbase(p, tile, k0) (wave-uniform pointer to element (k0, 0) of the expert's
// matrix), ld(p) (elements per k-row) and ncols(p) (N); columns past N read column N - 8.
// Load instruction i of wave w fills LDS slots [64 (i NW + w), + 64): k-rows RPI (i NW + w)
// + lane / CPR, 16-byte chunk c of a row at position c ^ tr_swz(row).
template <class C, class Src, class P>
struct KMajorRowsB {
  static constexpr int CPR = C::BN / 8;                 // 16-byte chunks per k-row
  static constexpr int RPI = 64 / CPR;                  // k-rows per load instruction
  static constexpr int INST = C::BK * CPR / 64;
  static constexpr int PER = INST / C::NW;
  static_assert(CPR >= 16 && 64 % CPR == 0 && INST % C::NW == 0 && (RPI * C::NW) % 4 == 0, "k-major B tile");
  uint32_t colb;                                        // byte offset of this lane's chunk in a k-row
  int rsub;
  __device__ void init(const P& p, const Tile& tl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    rsub = lane / CPR;
    const int r = RPI * wave + rsub;                    // this lane's rows are r mod 4 for every i
    const int chunk = (lane % CPR) ^ tr_swz(r);
    colb = (uint32_t)min(tl.n0 + chunk * 8, Src::ncols(p) - 8) * 2u;
  }
  __device__ void issue_one(const P& p, const Tile& tl, int k0, uint4* lds, int i) const {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = (i * C::NW + wave) * 64;
    const uint8_t* b = reinterpret_cast<const uint8_t*>(Src::kbase(p, tl, k0));
    lds_dma16(b, (uint32_t)(S / CPR + rsub) * (uint32_t)Src::ld(p) * 2u + colb, lds_addr(lds + S));
  }
  __device__ void issue(const P& p, const Tile& tl, int k0, uint4* lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) issue_one(p, tl, k0, lds, i);
  }
};

// Byte offsets of this lane's MFMA operand chunks inside a stage, for sub-step 0.
// Chunk c of row r sits at position c ^ swz(r); a lane of half h reads chunk
// 2 kk + h = (2 kk) ^ h at sub-step kk, so its position is (swz(r) ^ h) ^ 2 kk and
// the byte offset is base ^ (32 kk): one XOR per read, no per-sub-step table.
// With BKM the B tile is k-major (KMajorRowsB) and b[] are its transpose-read offsets.
template <class C, bool BKM = false>
struct FragAddr {
  uint32_t a[C::FM], b[C::FN];
  __device__ void init(int wm, int wn, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int r = wm * C::WTM + fm * 32 + (lane & 31);
      a[fm] = (uint32_t)(r * C::CPR + (swz<C::CPR>(r) ^ h)) * 16u;
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      if constexpr (BKM) {
        b[fn] = (uint32_t)C::A_SLOTS * 16u + tr_offset(wn * C::WTN + fn * 32, C::BN, lane);
      } else {
        const int r = wn * C::WTN + fn * 32 + (lane & 31);
        b[fn] = (uint32_t)(C::A_SLOTS + r * C::CPR + (swz<C::CPR>(r) ^ h)) * 16u;
      }
    }
  }
};

// One k-tile: BK / 16 MFMA sub-steps, the operand reads of sub-step kk + 1 in
// flight under the MFMAs of sub-step kk (two register sets).  With LOADS, the
// NLOAD global->LDS load instructions of a later k-tile (issue(j), j < NLOAD)
// are spread over the sub-steps, one between two MFMAs, so that no wave stalls
// on a burst of vector-memory issues before its MFMAs.
// The A operand is read at sa + fa.a and B at sb + fa.b; fa.b counts from the start of a
// two-operand stage (A first), so for separate stages sb is the B stage less the A part's bytes.
template <class C, bool LOADS, int NLOAD, bool BKM, class Issue>
__device__ __forceinline__ void mma_ktile_rows(const uint8_t* sa, const uint8_t* sb, const FragAddr<C, BKM>& fa,
                                               f32x16 (&acc)[C::FM][C::FN], Issue issue) {
  constexpr int KK = C::BK / 16;
  constexpr int NR = C::FM + (BKM ? 2 : 1) * C::FN, NM = C::FM * C::FN;
  constexpr int LPS = MOE_ROWS_LPS < NLOAD ? MOE_ROWS_LPS : NLOAD;   // loads per sub-step, front-loaded
  static_assert(!LOADS || LPS * KK >= NLOAD, "every load of the k-tile must be issued");
  bf16x8 a[2][C::FM], b[2][C::FN];
  auto load = [&](int kk, int buf) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
      a[buf][fm] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sa + (fa.a[fm] ^ (32u * kk))));
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      if constexpr (BKM)
        b[buf][fn] = tr_frag((const lds_u8*)sb, fa.b[fn] + 16u * kk * (C::BN * 2), C::BN * 2);
      else
        b[buf][fn] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(sb + (fa.b[fn] ^ (32u * kk))));
    }
  };
  load(0, 0);
  static_for<0, KK>([&](auto kkc) {
    constexpr int kk = decltype(kkc)::value;
    constexpr int J0 = kk * LPS, J1 = (kk + 1) * LPS < NLOAD ? (kk + 1) * LPS : NLOAD;
    constexpr int NL = LOADS && J1 > J0 ? J1 - J0 : 0;
    if constexpr (kk + 1 < KK) load(kk + 1, (kk + 1) & 1);
    static_for<0, NL>([&](auto jc) { issue(J0 + decltype(jc)::value); });
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[kk & 1][fn], a[kk & 1][fm], acc[fm][fn], 0, 0, 0);
    // issue order: the next sub-step's LDS reads early, between the first MFMAs,
    // then the global loads one per MFMA
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most `pending` k-tiles (of P instructions each, per wave) are outstanding.
template <int NST, int P>
__device__ __forceinline__ void wait_ktiles(int pending) {
  if constexpr (NST >= 4) {
    if (pending >= 2) { wait_vmcnt<2 * P>(); return; }
  }
  if constexpr (NST >= 3) {
    if (pending >= 1) { wait_vmcnt<P>(); return; }
  }
  wait_vmcnt<0>();
}

// Body: Ops provides Sched (RowGroups), SrcA, SrcB, init_sched() and
// epilogue(p, tile, acc, wm, wn, lane, wave_lds): wave_lds is a private LDS
// scratch of EPI_BYTES bytes per wave (the stage the next tile's prologue does
// not use) for staging the output tile into whole-row stores.
template <class C>
struct RowEpiLds {
  static constexpr int BYTES = C::EPI;
};

// LDS of the schedule: prefix of per-expert tile counts (up to 1024 experts) and the
// block scan's partial sums.
constexpr int SCHED_LDS_INTS = 1024 + 1 + 16 + 1;

// Whether Ops' B operand is k-major (Ops::B_KMAJOR, false when absent): loaded by KMajorRowsB
// and read with transpose reads.
template <class T, class = void>
struct BKMajor : std::false_type {};
template <class T>
struct BKMajor<T, std::void_t<decltype(T::B_KMAJOR)>> : std::bool_constant<T::B_KMAJOR> {};

// Whether Ops takes the two-stage schedule that issues the next tile's first k-tile in the
// last k step (Ops::EARLY_NEXT, true when absent): an epilogue that already needs every
// register keeps the plain schedule.
template <class T, class = void>
struct EarlyNext : std::true_type {};
template <class T>
struct EarlyNext<T, std::void_t<decltype(T::EARLY_NEXT)>> : std::bool_constant<T::EARLY_NEXT> {};

// Output stores per wave and tile that Ops' epilogue issues whatever the tile's rows
// (Ops::OUT_STORES, -1 when absent: not counted), and whether it did so for these arguments
// (Ops::stores_counted(p)).
template <class T, class = void>
struct OutStores : std::integral_constant<int, -1> {};
template <class T>
struct OutStores<T, std::void_t<decltype(T::OUT_STORES)>> : std::integral_constant<int, T::OUT_STORES> {};

// Every tile of Ops' schedule, with the stages at smem (C::NST * C::STAGE uint4) and the
// schedule's scratch at sched_lds.  `carry` is XcdWalk's deal position, updated for a
// schedule that follows on the same grid.
// With LT the schedule's scratch is the stage area (sched_lds is not used) and the workgroup's
// tiles come from a lane table built when the pass starts (the launch gives no workgroup more
// than LANE_TILES tiles of a pass).
template <class C, class Ops, class P, bool LT = false>
__device__ __forceinline__ void rows_gemm_tiles(const P& p, uint4* smem, int* sched_lds, int& carry) {
  static_assert(C::NT / 64 <= 16, "schedule scratch");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  constexpr bool BKM = BKMajor<Ops>::value;
  using AL = DirectRows<C, C::BM, typename Ops::SrcA, P>;
  using BL = std::conditional_t<BKM, KMajorRowsB<C, typename Ops::SrcB, P>, DirectRows<C, C::BN, typename Ops::SrcB, P>>;
  constexpr int PERK = AL::PER + BL::PER;                 // real load instructions per k-tile per wave

  typename Ops::Sched sched;
  int* pre = LT ? reinterpret_cast<int*>(smem) : sched_lds;
  Ops::init_sched(sched, p, pre, pre + 1025);
  XcdWalk walk;
  carry = walk.init(sched.total, carry);
  LaneTiles<typename Ops::Sched> lt;
  int ntile;
  if constexpr (LT) {
    lt.init(sched, walk.t, walk.step, walk.end);
    ntile = lt.n;
    __syncthreads();                                      // the prefix is read before loads land on it
  } else {
    ntile = walk.t < walk.end ? (walk.end - walk.t + walk.step - 1) / walk.step : 0;
  }
  if (ntile == 0) return;
  auto tile_at = [&](int i) {
    if constexpr (LT) return lt.get(sched, i);
    else return sched.tile(walk.t + i * walk.step);
  };
  int ti = 0;                                             // the current tile's index
  Tile tl = tile_at(0);
  FragAddr<C, BKM> fa;
  fa.init(wm, wn, lane);
  AL al;
  BL bl;
  al.init(p, tl);
  bl.init(p, tl);
  int nk = (tl.k_hi - tl.k_lo) / C::BK;
  // prologue: first NST-1 k-tiles of the first tile
#pragma unroll
  for (int s = 0; s < C::NST - 1; ++s)
    if (s < nk) {
      al.issue(p, tl, s * C::BK, smem + s * C::STAGE);
      bl.issue(p, tl, s * C::BK, smem + s * C::STAGE + C::A_SLOTS);
    }
  if constexpr (C::NST == 2 && EarlyNext<Ops>::value) {
    // Two stages: the last k step of a tile issues the next tile's first k-tile into the
    // other stage, the epilogue waits for it (one k step old) before its output stores and
    // uses the stage just read as scratch, and the next tile's first k step needs no wait.
    // The output stores then drain under that k step and are only waited for at the second
    // one, instead of stalling every workgroup at the tile boundary.
    int base = 0;                                         // stage of k-tile 0 of the current tile
    bool prewaited = false;                               // k-tile 0 already waited for
    while (true) {
      f32x16 acc[C::FM][C::FN];
#pragma unroll
      for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
      const Tile cur_tile = tl;
      for (int kt = 0; kt < nk - 1; ++kt) {
        if (kt > 0 || !prewaited) wait_vmcnt<0>();
        __syncthreads();
        const int cs = (base + kt) & 1;
        uint4* st = smem + (cs ^ 1) * C::STAGE;
        const int k0 = (kt + 1) * C::BK;
        auto issue = [&](int j) {
          if (j < AL::PER) al.issue_one(p, cur_tile, k0, st, j);
          else bl.issue_one(p, cur_tile, k0, st + C::A_SLOTS, j - AL::PER);
        };
        const uint8_t* cst = reinterpret_cast<const uint8_t*>(smem + cs * C::STAGE);
        mma_ktile_rows<C, true, PERK, BKM>(cst, cst, fa, acc, issue);
      }
      // last k step: its loads are the next tile's first k-tile
      if (nk > 1 || !prewaited) wait_vmcnt<0>();
      __syncthreads();
      const int scratch = (base + nk - 1) & 1;            // the stage this step reads
      const bool more = ++ti < ntile;
      {
        // without a next tile the same loads fetch this tile's first k-tile again (in bounds,
        // never read), so that the MFMA sequence has no branch around it
        tl = more ? tile_at(ti) : cur_tile;
        al.init(p, tl);
        bl.init(p, tl);
        uint4* st = smem + (scratch ^ 1) * C::STAGE;
        auto issue = [&](int j) {
          if (j < AL::PER) al.issue_one(p, tl, 0, st, j);
          else bl.issue_one(p, tl, 0, st + C::A_SLOTS, j - AL::PER);
        };
        const uint8_t* sst = reinterpret_cast<const uint8_t*>(smem + scratch * C::STAGE);
        mma_ktile_rows<C, true, PERK, BKM>(sst, sst, fa, acc, issue);
      }
      // every wave is past its last LDS read before the stage it read becomes scratch
      __syncthreads();
      wait_vmcnt<0>();                                    // the next tile's first k-tile (or the
                                                          // unread reload: no LDS write may be
                                                          // in flight when the workgroup ends)
      uint8_t* wave_lds = reinterpret_cast<uint8_t*>(smem + scratch * C::STAGE) + wave * RowEpiLds<C>::BYTES;
      Ops::epilogue(p, cur_tile, acc, wm, wn, lane, wave_lds);
      if (!more) break;
      // the scratch stage receives the next tile's second k-tile: all waves must be done with it
      __syncthreads();
      base = scratch ^ 1;
      nk = (tl.k_hi - tl.k_lo) / C::BK;
      prewaited = true;
    }
  } else {
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
        const int ahead = nk - 1 - kt;                      // k-tiles issued after this one (capped)
        if (kt == 0) wait_vmcnt<0>();
        else wait_ktiles<C::NST, PERK>(ahead < C::NST - 2 ? ahead : C::NST - 2);
        __syncthreads();
        const int nxt = kt + C::NST - 1;
        uint4* st = smem + (nxt % C::NST) * C::STAGE;
        auto issue = [&](int j) {
          if (j < AL::PER) al.issue_one(p, tl, nxt * C::BK, st, j);
          else bl.issue_one(p, tl, nxt * C::BK, st + C::A_SLOTS, j - AL::PER);
        };
        const uint8_t* cur = reinterpret_cast<const uint8_t*>(smem + (kt % C::NST) * C::STAGE);
        mma_ktile_rows<C, decltype(loads)::value, PERK, BKM>(cur, cur, fa, acc, issue);
      };
      // the last NST - 1 k steps issue nothing: peeled, not branched, so that the
      // two instantiations never meet inside one loop body
      int kt = 0;
      for (; kt < nk - (C::NST - 1); ++kt) kstep(kt, std::true_type{});
      for (; kt < nk; ++kt) kstep(kt, std::false_type{});
      // every wave is past its last LDS read before any stage is refilled
      __syncthreads();
      const Tile done = tl;
      const bool more = ++ti < ntile;
      if (more) {
        // start the next tile's loads, then run this tile's epilogue under them
        tl = tile_at(ti);
        al.init(p, tl);
        bl.init(p, tl);
        nk = (tl.k_hi - tl.k_lo) / C::BK;
#pragma unroll
        for (int s = 0; s < C::NST - 1; ++s)
          if (s < nk) {
            al.issue(p, tl, s * C::BK, smem + s * C::STAGE);
            bl.issue(p, tl, s * C::BK, smem + s * C::STAGE + C::A_SLOTS);
          }
      }
      uint8_t* wave_lds = reinterpret_cast<uint8_t*>(smem + (C::NST - 1) * C::STAGE) + wave * RowEpiLds<C>::BYTES;
      Ops::epilogue(p, done, acc, wm, wn, lane, wave_lds);
      if (!more) break;
      // the scratch stage is the next tile's last stage: all waves must be done with it
      __syncthreads();
    }
  }
}

template <class C, class Ops, class P>
__device__ __forceinline__ void rows_gemm_body(const P& p) {
  __shared__ uint4 smem[C::NST * C::STAGE];
  __shared__ int sched_lds[SCHED_LDS_INTS];
  int carry = 0;
  rows_gemm_tiles<C, Ops, P>(p, smem, sched_lds, carry);
}

// The full-tile pass with the weight operand requested two k steps ahead: two A stages and three
// B stages, [A0 | A1 | B0 | B1 | B2] (2 x 32 KB + 3 x 32 KB = 160 KB for 256 x 256 x 64 tiles),
// and the row operand one k step ahead.  k-tiles are numbered g over the workgroup's tiles (nk per
// tile; A k-tile g in A stage g mod 2, B k-tile g in B stage g mod 3).  Step g waits for A and B
// k-tile g, then issues A k-tile g + 1 and B k-tile g + 2 (the A loads first, so that waiting for
// all but the last PB loads leaves only B k-tile g + 2 in flight); loads past the workgroup's last
// tile fetch its last k-tile 0 again (in bounds, never read).
// At a tile's end (g = the next tile's first k-tile) the A stage and the B stage just read are
// free: A k-tile g + 1 is issued at once into the A one, the epilogue waits for A and B k-tile g,
// stages its output in the B one and issues its stores, and the next tile's first step issues
// only B k-tile g + 2 (into the staging area, after a barrier).  With an epilogue whose stores
// are counted (OutStores), the second step waits for A and B k-tile g + 1 but lets the SO stores
// issued after them stay in flight, so they drain under two k steps; otherwise it waits for
// them.  The schedule's prefix and the tile lookups use the stage area before the first load
// (lane table).  A gathered row operand's loader loads its token ids when it moves to the next
// tile; the compiler waits for those loads with vmcnt(0), which also drains the k-tiles in
// flight, once per tile.
template <class C, class Ops, class P>
__device__ __forceinline__ void rows_gemm_tiles_db(const P& p, uint4* smem, int& carry) {
  static_assert(C::NST == 2 && C::BM == C::BN && EarlyNext<Ops>::value, "two stages, square tiles");
  static_assert(C::EPI * C::NW <= C::B_SLOTS * 16, "epilogue staging inside one B stage");
  constexpr int SO = OutStores<Ops>::value;               // counted output stores per wave (-1: none)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  constexpr bool BKM = BKMajor<Ops>::value;
  using AL = DirectRows<C, C::BM, typename Ops::SrcA, P>;
  using BL = std::conditional_t<BKM, KMajorRowsB<C, typename Ops::SrcB, P>, DirectRows<C, C::BN, typename Ops::SrcB, P>>;
  constexpr int PA = AL::PER, PB = BL::PER, PERK = PA + PB;
  uint4* const As = smem;                                 // A stage s: As + s * A_SLOTS
  uint4* const Bs = smem + 2 * C::A_SLOTS;                // B stage s: Bs + s * B_SLOTS

  typename Ops::Sched sched;
  int* pre = reinterpret_cast<int*>(smem);
  Ops::init_sched(sched, p, pre, pre + 1025);
  XcdWalk walk;
  carry = walk.init(sched.total, carry);
  LaneTiles<typename Ops::Sched> lt;
  lt.init(sched, walk.t, walk.step, walk.end);
  const int ntile = lt.n;
  __syncthreads();                                        // the prefix is read before loads land on it
  if (ntile == 0) return;
  FragAddr<C, BKM> fa;
  fa.init(wm, wn, lane);

  // load cursors: the tile and k-tile each operand's next load fetches
  Tile ta = lt.get(sched, 0), tb = ta;
  const int nk = (ta.k_hi - ta.k_lo) / C::BK;             // the same for every tile of the pass
  int ia = 0, ka = 0, ib = 0, kb = 0;
  AL al;
  BL bl;
  al.init(p, ta);
  bl.init(p, tb);
  auto next_a = [&]() {
    if (++ka == nk) {
      ka = 0;
      if (ia + 1 < ntile) {
        ta = lt.get(sched, ++ia);
        al.init(p, ta);
      }
    }
  };
  auto next_b = [&]() {
    if (++kb == nk) {
      kb = 0;
      if (ib + 1 < ntile) {
        tb = lt.get(sched, ++ib);
        bl.init(p, tb);
      }
    }
  };
  // prologue: A k-tile 0, B k-tiles 0 and 1
  al.issue(p, ta, 0, As);
  next_a();
  bl.issue(p, tb, 0, Bs);
  next_b();
  bl.issue(p, tb, kb * C::BK, Bs + C::B_SLOTS);
  next_b();
  int g = 0;                                              // the k-tile the next step computes
  bool after_epi = false;                                 // an epilogue ran before this tile
  bool counted = false;                                   // ... and its SO stores are in flight
  for (int ti = 0; ti < ntile; ++ti) {
    const Tile cur = lt.get(sched, ti);
    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
    for (int k = 0; k < nk; ++k, ++g) {
      // (after an epilogue: step 0's k-tiles were waited for at the tile's end; step 1's were
      // issued before the epilogue's stores)
      if (!after_epi || k > 1) wait_vmcnt<PB>();
      else if (k == 1) {
        if constexpr (SO >= 0) {
          if (counted) wait_vmcnt<PB + SO>();
          else wait_vmcnt<PB>();
        } else {
          wait_vmcnt<PB>();
        }
      }
      __syncthreads();
      uint4* sta = As + ((g + 1) & 1) * C::A_SLOTS;
      uint4* stb = Bs + ((g + 2) % 3) * C::B_SLOTS;
      const int k0a = ka * C::BK, k0b = kb * C::BK;
      const uint8_t* sa = reinterpret_cast<const uint8_t*>(As + (g & 1) * C::A_SLOTS);
      const uint8_t* sb = reinterpret_cast<const uint8_t*>(Bs + (g % 3) * C::B_SLOTS) - C::A_SLOTS * 16;
      if (after_epi && k == 0) {
        // A k-tile g + 1 is already in flight: B only
        auto issue = [&](int j) { bl.issue_one(p, tb, k0b, stb, j); };
        mma_ktile_rows<C, true, PB, BKM>(sa, sb, fa, acc, issue);
      } else {
        auto issue = [&](int j) {
          if (j < PA) al.issue_one(p, ta, k0a, sta, j);
          else bl.issue_one(p, tb, k0b, stb, j - PA);
        };
        mma_ktile_rows<C, true, PERK, BKM>(sa, sb, fa, acc, issue);
        next_a();
      }
      next_b();
    }
    // every wave is past its reads of the A and B stages of the last step
    __syncthreads();
    // A k-tile g + 1 into the A stage just read, then wait for A and B k-tile g (B k-tile g + 1
    // and A k-tile g + 1 stay in flight)
    al.issue(p, ta, ka * C::BK, As + ((g + 1) & 1) * C::A_SLOTS);
    next_a();
    wait_vmcnt<PB + PA>();
    after_epi = true;
    if constexpr (SO >= 0) counted = Ops::stores_counted(p);
    // the output stores follow those loads in issue order
    asm volatile("" ::: "memory");
    uint8_t* wave_lds = reinterpret_cast<uint8_t*>(Bs + ((g + 2) % 3) * C::B_SLOTS) + wave * C::EPI;
    Ops::epilogue(p, cur, acc, wm, wn, lane, wave_lds);
    // the staging area receives the next step's B load
    __syncthreads();
  }
  wait_vmcnt<0>();                                        // no LDS write in flight when the pass ends
}

// Four passes over the experts' rows in one kernel, sharing one LDS allocation:
// the full 256-row tiles (and remainders above 192 rows) with configuration CF,
// then each remainder of at most 192, 128 and 64 rows in one C3, C2 or C1 tile.
// A workgroup that is done with its share of one pass goes on to its share of
// the next.
template <int A, int B>
constexpr int cmax() { return A > B ? A : B; }
template <class CF, class C3, class C2, class C1, class OpsF, class Ops3, class Ops2, class Ops1, class P>
__device__ __forceinline__ void rows_gemm_split_body(const P& p) {
  static_assert(C3::NT == CF::NT && C2::NT == CF::NT && C1::NT == CF::NT, "one block shape");
  constexpr int SMAX = cmax<cmax<CF::NST * CF::STAGE, C3::NST * C3::STAGE>(),
                           cmax<C2::NST * C2::STAGE, C1::NST * C1::STAGE>()>();
  __shared__ uint4 smem[SMAX];
  __shared__ int sched_lds[SCHED_LDS_INTS];
  int carry = 0;
  rows_gemm_tiles<CF, OpsF, P>(p, smem, sched_lds, carry);
  __syncthreads();
  rows_gemm_tiles<C3, Ops3, P>(p, smem, sched_lds, carry);
  __syncthreads();
  rows_gemm_tiles<C2, Ops2, P>(p, smem, sched_lds, carry);
  __syncthreads();
  rows_gemm_tiles<C1, Ops1, P>(p, smem, sched_lds, carry);
}

// The four passes with the full-tile pass on the deep-B schedule (rows_gemm_tiles_db) and the
// remainder passes on lane tables, all in one LDS allocation with no schedule scratch beside it.
template <class CF, class C3, class C2, class C1, class OpsF, class Ops3, class Ops2, class Ops1, class P>
__device__ __forceinline__ void rows_gemm_split_body_db(const P& p) {
  static_assert(C3::NT == CF::NT && C2::NT == CF::NT && C1::NT == CF::NT, "one block shape");
  constexpr int SDB = 2 * CF::A_SLOTS + 3 * CF::B_SLOTS;
  constexpr int SMAX = cmax<cmax<SDB, C3::NST * C3::STAGE>(), cmax<C2::NST * C2::STAGE, C1::NST * C1::STAGE>()>();
  __shared__ uint4 smem[SMAX];
  int carry = 0;
  rows_gemm_tiles_db<CF, OpsF, P>(p, smem, carry);
  __syncthreads();
  rows_gemm_tiles<C3, Ops3, P, true>(p, smem, nullptr, carry);
  __syncthreads();
  rows_gemm_tiles<C2, Ops2, P, true>(p, smem, nullptr, carry);
  __syncthreads();
  rows_gemm_tiles<C1, Ops1, P, true>(p, smem, nullptr, carry);
}

// Output stores through a buffer resource (raw buffer: stride 0; the hardware drops a store
// whose offset is at or past the resource's size).  Every wave issues every such store,
// whether or not any of its lanes is in range, so the number of vector-memory operations an
// epilogue leaves in flight is a compile-time constant, which the deep-B schedule counts in the
// waits of the next tile's second k step.
constexpr uint32_t BUF_DROP = 0x80000000u;              // an offset past every output resource
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const void* base, uint32_t bytes) {
  const uint8_t* b = uniform_ptr(reinterpret_cast<const uint8_t*>(base));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes < 0x7fffffffu ? bytes : 0x7fffffffu);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(b), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t x, uint32_t y,
                                            uint32_t z, uint32_t w) {
  __builtin_amdgcn_raw_buffer_store_b128(u32x4nt{x, y, z, w}, r, off, 0, 0);
}
// Store instructions per wave of stage_store_bf16<C, CW, ...> with COUNTED.
template <class C, int CW>
constexpr int stage_store_count() { return C::FM * (32 * (CW * 2 / 16) / 64); }

// Stages this wave's bf16 output, one 32-row fragment row-block at a time,
// through its LDS scratch and writes whole row segments (16 bytes per lane,
// CW * 2 contiguous bytes per row).  val(fm, fn, q, j) gives the value of
// accumulator item 4q + j of fragment (fm, fn); col_of(fn, q) the column (in the
// wave's CW-wide slab) of that item group for lane half 0 (lane half 1 adds 4).
// NQ item groups per fragment are stored.  NT marks the global stores non-temporal (streamed
// through L2 without displacing the operand tiles other workgroups are still reading).
// COUNTED issues exactly stage_store_count<C, CW>() buffer stores per wave (rows at or past
// row_end and columns at or past ncols dropped by the resource's range); row0 and col0 are then
// the wave's first row and column.
template <class C, int CW, int NQ, bool NT = false, bool COUNTED = false, class Val, class Col>
__device__ __forceinline__ void stage_store_bf16(uint8_t* wlds, uint16_t* out, int ld, int row0, int row_end,
                                                 int col0, int ncols, int lane_, Val val, Col col_of) {
  static_assert(!(NT && COUNTED), "counted stores are plain");
  const int lane = opaque_lane(lane_);
  constexpr int CPRW = CW * 2 / 16;                      // 16-byte chunks per row
  // Rows padded by 16 bytes where the scratch allows it, else unpadded 128-byte
  // rows with chunk c of row r stored at c ^ ((r >> 1) & 7).
  constexpr bool SWZ = 32 * (CW * 2 + 16) > RowEpiLds<C>::BYTES;
  constexpr int PITCH = SWZ ? CW * 2 : CW * 2 + 16;
  static_assert(32 * PITCH <= RowEpiLds<C>::BYTES, "staging area too small");
  static_assert(!SWZ || CPRW == 8, "swizzled staging needs 128-byte rows");
  auto pos = [](int r, int ch) { return SWZ ? (ch ^ ((r >> 1) & 7)) : ch; };
  __amdgpu_buffer_rsrc_t rs;
  if constexpr (COUNTED) {
    const int valid = min(max(row_end - row0, 0), C::FM * 32);
    rs = out_rsrc(out + (size_t)row0 * ld + col0, (uint32_t)valid * (uint32_t)ld * 2u);
  }
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int r = lane & 31;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int c = col_of(fn, q) + (lane >> 5) * 4;
        uint2 v;
        v.x = pack_bf16x2(val(fm, fn, q, 0), val(fm, fn, q, 1));
        v.y = pack_bf16x2(val(fm, fn, q, 2), val(fm, fn, q, 3));
        *reinterpret_cast<uint2*>(wlds + r * PITCH + pos(r, c >> 3) * 16 + (c & 7) * 2) = v;
      }
    // read back 16-byte chunks: 64 / CPRW rows per step
#pragma unroll
    for (int i = 0; i < 32 * CPRW / 64; ++i) {
      const int idx = i * 64 + lane;
      const int rr = idx / CPRW, ch = idx % CPRW;
      const uint4 v = *reinterpret_cast<const uint4*>(wlds + rr * PITCH + pos(rr, ch) * 16);
      const int grow = row0 + fm * 32 + rr;
      const int gcol = col0 + ch * 8;
      if constexpr (COUNTED) {
        const uint32_t off = gcol < ncols ? ((uint32_t)(fm * 32 + rr) * (uint32_t)ld + ch * 8) * 2u : BUF_DROP;
        buf_store16(rs, off, v.x, v.y, v.z, v.w);
      } else if (grow < row_end && gcol < ncols) {
        uint16_t* dst = out + (size_t)grow * ld + gcol;
        if constexpr (NT)
          __builtin_nontemporal_store(u32x4nt{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4nt*>(dst));
        else
          *reinterpret_cast<uint4*>(dst) = v;
      }
    }
  }
}

// Writes this wave's bf16 output straight from the accumulators (no LDS staging): for each
// fragment row-block, lane l stores its row (l % 32) and, per item group, the four consecutive
// columns of its lane half (8 bytes; the two halves fill 16 contiguous bytes).  val and col_of as
// for stage_store_bf16; NT marks the stores non-temporal.
template <class C, int NQ, bool NT = false, class Val, class Col>
__device__ __forceinline__ void direct_store_bf16(uint16_t* out, int ld, int row0, int row_end, int col0, int ncols,
                                                  int lane, Val val, Col col_of) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int r = row0 + fm * 32 + (lane & 31);
    if (r >= row_end) continue;
    uint16_t* orow = out + (size_t)r * ld + col0 + (lane >> 5) * 4;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int c = col_of(fn, q);
        if (col0 + c + (lane >> 5) * 4 >= ncols) continue;
        const uint32_t x = pack_bf16x2(val(fm, fn, q, 0), val(fm, fn, q, 1));
        const uint32_t y = pack_bf16x2(val(fm, fn, q, 2), val(fm, fn, q, 3));
        if constexpr (NT)
          __builtin_nontemporal_store(u32x2nt{x, y}, reinterpret_cast<u32x2nt*>(orow + c));
        else
          *reinterpret_cast<uint2*>(orow + c) = make_uint2(x, y);
      }
  }
}

}  // namespace moe
