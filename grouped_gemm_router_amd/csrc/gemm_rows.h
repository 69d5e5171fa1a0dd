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

#include "grouped_gemm.h"

namespace moe {

template <int BM_, int BN_, int WAVES_M_, int WAVES_N_, int BK_, int NST_>
struct RowCfg {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, NW = WAVES_M_ * WAVES_N_;
  static constexpr int NT = 64 * NW;
  static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;
  static constexpr int FM = WTM / 32, FN = WTN / 32;
  static constexpr int BK = BK_, CPR = BK_ / 8, NST = NST_;
  static constexpr int A_SLOTS = BM * CPR, B_SLOTS = BN * CPR;      // 16-byte slots per stage
  static constexpr int STAGE = A_SLOTS + B_SLOTS;
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

// Loader of one operand: rows [0, ROWS) of the tile.  Src provides
//   static const uint16_t* base(const P&, const Tile&, int row0, int k0): wave-uniform base of the
//       rows [row0, row0 + 64 / CPR) for k-tile k0 (element 0 of the k-tile);
//   static uint32_t row_off(const P&, const Tile&, int row): element offset of the (clamped, valid)
//       row relative to that base.
template <class C, int ROWS, class Src, class P>
struct DirectRows {
  static constexpr int INST = ROWS * C::CPR / 64;        // load instructions per stage
  static constexpr int PER = INST / C::NW;               // ... per wave
  uint32_t off[PER];

  __device__ void init(const P& p, const Tile& tl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int s = (i * C::NW + wave) * 64 + lane;
      const int row = s / C::CPR;
      const int chunk = (s % C::CPR) ^ swz<C::CPR>(row);
      off[i] = Src::row_off(p, tl, row) + chunk * 8;
    }
  }
  // Issue the loads of k-tile k0 into the stage at `lds` (uint4 slots).
  __device__ void issue(const P& p, const Tile& tl, int k0, uint4* lds) const {
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int S = (i * C::NW + wave) * 64;
      const uint16_t* b = Src::base(p, tl, S / C::CPR, k0);
      __builtin_amdgcn_global_load_lds(b + off[i], lds + S, 16, 0, 0);
    }
  }
};

// L2 warming: one 16-byte load per tile row and k-tile, issued a few k-tiles
// ahead of the real loads into a dummy LDS slot.  Rows [0, BM) are operand A,
// [BM, BM + BN) operand B; lane l of wave w takes row w * 64 + l (and + NW * 64 ...).
// It is the newest vector-memory instruction of its k step, so the waits for the
// real loads (vmcnt is retired in issue order) never wait for it.
template <class C, class SrcA, class SrcB, class P>
struct RowPrefetch {
  static constexpr int ROWS = C::BM + C::BN;
  static constexpr int PER = (ROWS + 64 * C::NW - 1) / (64 * C::NW);
  __device__ static void issue(const P& p, const Tile& tl, int k0, uint4* dummy) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int row = (i * C::NW + wave) * 64 + lane;
      if (row < C::BM) {
        __builtin_amdgcn_global_load_lds(SrcA::base(p, tl, row, k0) + SrcA::row_off(p, tl, row), dummy, 16, 0, 0);
      } else if (row < ROWS) {
        const int rb = row - C::BM;
        __builtin_amdgcn_global_load_lds(SrcB::base(p, tl, rb, k0) + SrcB::row_off(p, tl, rb), dummy, 16, 0, 0);
      }
    }
  }
};

template <class C>
__device__ __forceinline__ void load_frags(const uint4* As, const uint4* Bs, int kk, int wm, int wn, int lane,
                                           bf16x8 (&a)[C::FM], bf16x8 (&b)[C::FN]) {
  const int ch = kk * 2 + (lane >> 5);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int r = wm * C::WTM + fm * 32 + (lane & 31);
    a[fm] = __builtin_bit_cast(bf16x8, As[r * C::CPR + (ch ^ swz<C::CPR>(r))]);
  }
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) {
    const int r = wn * C::WTN + fn * 32 + (lane & 31);
    b[fn] = __builtin_bit_cast(bf16x8, Bs[r * C::CPR + (ch ^ swz<C::CPR>(r))]);
  }
}

// One k-tile: BK / 16 MFMA sub-steps.  (Double-buffering the operand registers
// across sub-steps measured no faster: the loop is bound by global load latency.)
template <class C>
__device__ __forceinline__ void mma_ktile_rows(const uint4* As, const uint4* Bs, f32x16 (&acc)[C::FM][C::FN],
                                               int wm, int wn, int lane) {
#pragma unroll
  for (int kk = 0; kk < C::BK / 16; ++kk) {
    bf16x8 a[C::FM], b[C::FN];
    load_frags<C>(As, Bs, kk, wm, wn, lane, a, b);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[fn], a[fm], acc[fm][fn], 0, 0, 0);
  }
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
  static constexpr int BYTES = C::STAGE * 16 / C::NW;
};

template <class C, class Ops, class P>
__device__ __forceinline__ void rows_gemm_body(const P& p) {
  __shared__ uint4 smem[C::NST * C::STAGE];
  __shared__ uint4 dummy[64];
  __shared__ int sched_lds[1024 + 1 + C::NT / 64 + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  using AL = DirectRows<C, C::BM, typename Ops::SrcA, P>;
  using BL = DirectRows<C, C::BN, typename Ops::SrcB, P>;
  using PF = RowPrefetch<C, typename Ops::SrcA, typename Ops::SrcB, P>;
  constexpr int PERK = AL::PER + BL::PER;                 // real load instructions per k-tile per wave
  // L2 warming measured slower on the prefill and training shapes (extra requests and
  // in-order vmcnt waits on warming loads outweigh the misses they save): off.
  constexpr bool PREFETCH = false;
  constexpr int PF_DIST = 3;                              // k-tiles ahead of the one being computed

  typename Ops::Sched sched;
  Ops::init_sched(sched, p, sched_lds, sched_lds + 1025);
  XcdWalk walk;
  walk.init(sched.total);
  if (!walk.valid()) return;
  Tile tl = sched.tile(walk.t);
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
  if constexpr (PREFETCH) {
    for (int s = 1; s < PF_DIST && s < nk; ++s) PF::issue(p, tl, s * C::BK, dummy);
  }
  while (true) {
    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
    bool pf_last = false;                                 // did the previous k step issue a prefetch?
    for (int kt = 0; kt < nk; ++kt) {
      if constexpr (PREFETCH) {
        if (kt == 0) wait_vmcnt<0>();
        else if (pf_last) wait_vmcnt<1>();
        else wait_vmcnt<0>();
      } else {
        const int ahead = nk - 1 - kt;                    // k-tiles issued after this one (capped)
        if (kt == 0) wait_vmcnt<0>();
        else wait_ktiles<C::NST, PERK>(ahead < C::NST - 2 ? ahead : C::NST - 2);
      }
      __syncthreads();
      const int nxt = kt + C::NST - 1;
      if (nxt < nk) {
        uint4* st = smem + (nxt % C::NST) * C::STAGE;
        al.issue(p, tl, nxt * C::BK, st);
        bl.issue(p, tl, nxt * C::BK, st + C::A_SLOTS);
      }
      if constexpr (PREFETCH) {
        pf_last = kt + PF_DIST < nk;
        if (pf_last) PF::issue(p, tl, (kt + PF_DIST) * C::BK, dummy);
      }
      const uint4* cur = smem + (kt % C::NST) * C::STAGE;
      mma_ktile_rows<C>(cur, cur + C::A_SLOTS, acc, wm, wn, lane);
    }
    // every wave is past its last LDS read before any stage is refilled
    __syncthreads();
    const Tile done = tl;
    walk.next();
    const bool more = walk.valid();
    if (more) {
      // start the next tile's loads, then run this tile's epilogue under them
      tl = sched.tile(walk.t);
      al.init(p, tl);
      bl.init(p, tl);
      nk = (tl.k_hi - tl.k_lo) / C::BK;
#pragma unroll
      for (int s = 0; s < C::NST - 1; ++s)
        if (s < nk) {
          al.issue(p, tl, s * C::BK, smem + s * C::STAGE);
          bl.issue(p, tl, s * C::BK, smem + s * C::STAGE + C::A_SLOTS);
        }
      if constexpr (PREFETCH) {
        for (int s = 1; s < PF_DIST && s < nk; ++s) PF::issue(p, tl, s * C::BK, dummy);
      }
    }
    uint8_t* wave_lds = reinterpret_cast<uint8_t*>(smem + (C::NST - 1) * C::STAGE) + wave * RowEpiLds<C>::BYTES;
    Ops::epilogue(p, done, acc, wm, wn, lane, wave_lds);
    if (!more) break;
    // the scratch stage is the next tile's last stage: all waves must be done with it
    __syncthreads();
  }
}

// Stages this wave's bf16 output, one 32-row fragment row-block at a time,
// through its LDS scratch and writes whole row segments (16 bytes per lane,
// CW * 2 contiguous bytes per row).  val(fm, fn, q, j) gives the value of
// accumulator item 4q + j of fragment (fm, fn); col_of(fn, q) the column (in the
// wave's CW-wide slab) of that item group for lane half 0 (lane half 1 adds 4).
// NQ item groups per fragment are stored.
template <class C, int CW, int NQ, class Val, class Col>
__device__ __forceinline__ void stage_store_bf16(uint8_t* wlds, uint16_t* out, int ld, int row0, int row_end,
                                                 int col0, int ncols, int lane, Val val, Col col_of) {
  constexpr int PITCH = CW * 2 + 16;                     // bytes per staged row (16-byte aligned)
  constexpr int CPRW = CW * 2 / 16;                      // 16-byte chunks per row
  static_assert(32 * PITCH <= RowEpiLds<C>::BYTES, "staging area too small");
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
        *reinterpret_cast<uint2*>(wlds + r * PITCH + c * 2) = v;
      }
    // read back 16-byte chunks: 64 / CPRW rows per step
#pragma unroll
    for (int i = 0; i < 32 * CPRW / 64; ++i) {
      const int idx = i * 64 + lane;
      const int rr = idx / CPRW, ch = idx % CPRW;
      const uint4 v = *reinterpret_cast<const uint4*>(wlds + rr * PITCH + ch * 16);
      const int grow = row0 + fm * 32 + rr;
      const int gcol = col0 + ch * 8;
      if (grow < row_end && gcol < ncols) *reinterpret_cast<uint4*>(out + (size_t)grow * ld + gcol) = v;
    }
  }
}

}  // namespace moe
