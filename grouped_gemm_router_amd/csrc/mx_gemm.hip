// MXFP8 grouped GEMMs (gate/up + gated activation, down) on gfx950's block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and one E8M0 scale per
// 32 contraction elements of every row (OCP Microscaling v1.0).
//
// Same persistent row-group schedule, tile shape (256 x 256, 8 waves of
// 128 x 64) and direct global->LDS loads as the bf16 row GEMMs: a k-tile is
// 128 E4M3 codes, i.e. one 128-byte LDS row per tile row, exactly the bytes of
// a bf16 k-tile of 64, so the loader and the chunk swizzle are shared (the code
// arrays are addressed as 16-bit words).  Next to the data, each stage holds
// one 32-bit word per tile row with the row's four scale bytes of the k-tile,
// loaded by one dword-per-lane direct load per wave.
//
// Operand layout of the scaled MFMA (verified on the device): for a 64-long
// k chunk, lane half h (= lane / 32) supplies bytes [16h, 16h+16) and
// [32+16h, 32+16h+16) of its row, and its scale operand applies to the
// 32-element block [32h, 32h+32).  So MFMA kk of a k-tile reads 16-byte chunks
// 4kk+h and 4kk+2+h and scale byte 2kk+h.
#include "gemm_rows.h"
#include "kernels.h"

namespace moe {

// 256 x 256 tiles, k-tiles of 64 16-bit words (128 E4M3 codes), two stages
using CfgMx = RowCfg<256, 256, 2, 4, 64, 2>;

__device__ __forceinline__ int mx_clamp_row(const Tile& t, int row) { return min(t.m0 + row, t.m_end - 1); }

// Data sources (codes seen as 16-bit words: k0 and offsets count words) and the
// byte address of each row's first scale (scale k-tile kt is 4 bytes further per kt).
struct MxSrcX {        // gathered token rows of the quantised X
  static constexpr bool NARROW = true;   // scale rows: wave-uniform base + 32-bit offset
  __device__ static const uint16_t* base(const MxArgs& p, const Tile&, int, int k0) {
    return reinterpret_cast<const uint16_t*>(p.Xq) + k0;
  }
  __device__ static uint32_t row_off(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)p.row_token[mx_clamp_row(t, row)] * (uint32_t)(p.H / 2);
  }
  __device__ static const uint8_t* sbase(const MxArgs& p, const Tile&) { return p.Xs; }
  __device__ static uint32_t soff(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)p.row_token[mx_clamp_row(t, row)] * (uint32_t)(p.H / 32);
  }
};
// Packed gate / up codes [E, I, H], interleaved like the bf16 gate/up B tile:
// inside every 32-row MFMA fragment rows 0-15 are gate and rows 16-31 the up
// rows of the same 16 intermediate columns.
template <class C>
struct MxSrcGateUpW {
  __device__ static int col(const MxArgs& p, const Tile& t, int row) {
    return min(t.nt * (C::BN / 2) + (row / 32) * 16 + (row % 16), p.I - 1);
  }
  __device__ static const uint16_t* base(const MxArgs& p, const Tile& t, int row0, int k0) {
    const bool up = (row0 % 32) >= 16;
    return reinterpret_cast<const uint16_t*>(up ? p.Wu : p.Wg) + (size_t)t.e * p.I * (p.H / 2) + k0;
  }
  __device__ static uint32_t row_off(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)col(p, t, row) * (uint32_t)(p.H / 2);
  }
  // gate and up rows alternate inside a wave and their scales are separate arrays: a 64-bit
  // address per lane
  static constexpr bool NARROW = false;
  __device__ static const uint8_t* scales(const MxArgs& p, const Tile& t, int row) {
    const bool up = (row % 32) >= 16;
    return (up ? p.Su : p.Sg) + ((size_t)t.e * p.I + col(p, t, row)) * (p.H / 32);
  }
};
struct MxSrcUpW {      // packed up codes [E, I, H]: the B rows of the ungated (ReLU^2) up GEMM
  static constexpr bool NARROW = true;   // scale rows: wave-uniform base + 32-bit offset
  __device__ static const uint16_t* base(const MxArgs& p, const Tile& t, int, int k0) {
    return reinterpret_cast<const uint16_t*>(p.Wu) + (size_t)t.e * p.I * (p.H / 2) + k0;
  }
  __device__ static uint32_t row_off(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)min(t.n0 + row, p.I - 1) * (uint32_t)(p.H / 2);
  }
  __device__ static const uint8_t* sbase(const MxArgs& p, const Tile& t) { return p.Su + (size_t)t.e * p.I * (p.H / 32); }
  __device__ static uint32_t soff(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)min(t.n0 + row, p.I - 1) * (uint32_t)(p.H / 32);
  }
};
struct MxSrcH {        // expert-major quantised h rows
  static constexpr bool NARROW = true;   // scale rows: wave-uniform base + 32-bit offset
  __device__ static const uint16_t* base(const MxArgs& p, const Tile&, int, int k0) {
    return reinterpret_cast<const uint16_t*>(p.Hq) + k0;
  }
  __device__ static uint32_t row_off(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)mx_clamp_row(t, row) * (uint32_t)(p.I / 2);
  }
  __device__ static const uint8_t* sbase(const MxArgs& p, const Tile&) { return p.Hs; }
  __device__ static uint32_t soff(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)mx_clamp_row(t, row) * (uint32_t)(p.I / 32);
  }
};
struct MxSrcDownW {    // packed down codes [E, H, I]
  static constexpr bool NARROW = true;   // scale rows: wave-uniform base + 32-bit offset
  __device__ static const uint16_t* base(const MxArgs& p, const Tile& t, int, int k0) {
    return reinterpret_cast<const uint16_t*>(p.Wd) + (size_t)t.e * p.H * (p.I / 2) + k0;
  }
  __device__ static uint32_t row_off(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)min(t.n0 + row, p.H - 1) * (uint32_t)(p.I / 2);
  }
  __device__ static const uint8_t* sbase(const MxArgs& p, const Tile& t) { return p.Sd + (size_t)t.e * p.H * (p.I / 32); }
  __device__ static uint32_t soff(const MxArgs& p, const Tile& t, int row) {
    return (uint32_t)min(t.n0 + row, p.H - 1) * (uint32_t)(p.I / 32);
  }
};

// Scale words of the tile rows: 4 dword loads of 64 lanes per operand; wave w
// of group g (waves 0-3: A, 4-7: B) loads rows 64 w .. 64 w + 63 of its operand.
template <class SrcA, class SrcB>
struct MxScaleRows {
  static constexpr bool NARROW = SrcA::NARROW && SrcB::NARROW;
  const uint8_t* base;        // NARROW: wave-uniform base and this lane's 32-bit offset;
  uint32_t off;               // otherwise base is this lane's address (off unused)
  __device__ void init(const MxArgs& p, const Tile& tl, int wave) {
    const int row = (wave & 3) * 64 + opaque_lane(threadIdx.x & 63);
    // (a wave-uniform branch: a select between the two sources became a private array)
    off = 0;
    if (wave < 4) {
      if constexpr (NARROW) {
        base = SrcA::sbase(p, tl);
        off = SrcA::soff(p, tl, row);
      } else {
        base = scales_of<SrcA>(p, tl, row);
      }
    } else {
      if constexpr (NARROW) {
        base = SrcB::sbase(p, tl);
        off = SrcB::soff(p, tl, row);
      } else {
        base = scales_of<SrcB>(p, tl, row);
      }
    }
  }
  template <class S>
  __device__ static const uint8_t* scales_of(const MxArgs& p, const Tile& tl, int row) {
    if constexpr (S::NARROW) return S::sbase(p, tl) + S::soff(p, tl, row);
    else return S::scales(p, tl, row);
  }
  // this wave's 64 scale words of k-tile kt into lds (the operand's word array)
  __device__ void issue(int kt, uint32_t* lds, int wave) const {
    if constexpr (NARROW) {
      asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(off + (uint32_t)kt * 4u), "s"(uniform_ptr(base)),
                   "s"(lds_addr(lds + (wave & 3) * 64))
                   : "m0");
    } else {
      const uint8_t* a = base + (size_t)kt * 4;
      asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(a),
                   "s"(lds_addr(lds + (wave & 3) * 64))
                   : "m0");
    }
  }
};

// Byte offset of this lane's chunk 4kk + h of its row, for kk = 0 (chunk c of
// row r is at c ^ swz(r); chunk 4kk + 2 + h is at this ^ 32, kk = 1 at ^ 64).
template <class C>
struct MxFragAddr {
  uint32_t a[C::FM], b[C::FN];
  __device__ void init(int wm, int wn, int lane) {
    const int h = lane >> 5;
    const int ra = wm * C::WTM + (lane & 31);
    const int rb = wn * C::WTN + (lane & 31);
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int r = ra + fm * 32;
      a[fm] = (uint32_t)(r * C::CPR + (swz<C::CPR>(r) ^ h)) * 16u;
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int r = rb + fn * 32;
      b[fn] = (uint32_t)(C::A_SLOTS + r * C::CPR + (swz<C::CPR>(r) ^ h)) * 16u;
    }
  }
};

__device__ __forceinline__ i32x8 mx_operand(const uint8_t* stage, uint32_t off, int kk) {
  const uint4 lo = *reinterpret_cast<const uint4*>(stage + (off ^ (64u * kk)));
  const uint4 hi = *reinterpret_cast<const uint4*>(stage + (off ^ (64u * kk + 32u)));
  return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// One k-tile: two 64-wide MFMA steps, each over both B fragments and the A
// fragments two at a time; with LOADS the NLOAD direct loads of the next
// k-tile (issue(j)) are issued with the first step.
template <class C, bool LOADS, int NLOAD, class Issue>
__device__ __forceinline__ void mma_ktile_mx(const uint8_t* stage, const uint32_t* sA, const uint32_t* sB,
                                             const MxFragAddr<C>& fa, f32x16 (&acc)[C::FM][C::FN], int lane,
                                             Issue issue) {
  const int h = lane >> 5;
  uint32_t wa[C::FM], wb[C::FN];
  // the scale rows of this lane's fragments, recomputed here rather than held across the kernel
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ra = (wave / C::WAVES_N) * C::WTM + (opaque_lane(lane) & 31);
  const int rb = (wave % C::WAVES_N) * C::WTN + (opaque_lane(lane) & 31);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) wa[fm] = sA[ra + 32 * fm];
#pragma unroll
  for (int fn = 0; fn < C::FN; ++fn) wb[fn] = sB[rb + 32 * fn];
  static_for<0, 2>([&](auto kkc) {
    constexpr int kk = decltype(kkc)::value;
    const int sh = 8 * (2 * kk + h);
    i32x8 b[C::FN];
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) b[fn] = mx_operand(stage, fa.b[fn], kk);
    if constexpr (LOADS && kk == 0) static_for<0, NLOAD>([&](auto jc) { issue(decltype(jc)::value); });
    static_for<0, C::FM / 2>([&](auto pc) {
      constexpr int f0 = 2 * decltype(pc)::value;
      const i32x8 a0 = mx_operand(stage, fa.a[f0], kk), a1 = mx_operand(stage, fa.a[f0 + 1], kk);
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn) {
        const int sbn = (int)((wb[fn] >> sh) & 0xffu);
        acc[f0][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[fn], a0, acc[f0][fn], 0, 0, 0, sbn, 0,
                                                                      (int)((wa[f0] >> sh) & 0xffu));
        acc[f0 + 1][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            b[fn], a1, acc[f0 + 1][fn], 0, 0, 0, sbn, 0, (int)((wa[f0 + 1] >> sh) & 0xffu));
      }
      __builtin_amdgcn_sched_barrier(0);
    });
  });
}

// Persistent body (two stages; the bf16 row GEMM's pipeline with the scale
// words added).  Waves 0-3 load the A scales, waves 4-7 the B scales.
template <class C, class SrcA, class SrcB, class Epi, int GROUP_M = 1>
__device__ __forceinline__ void mx_rows_body(const MxArgs& p, int N, int K) {
  __shared__ uint4 smem[2 * C::STAGE];
  __shared__ uint32_t sscale[2][C::BM + C::BN];
  __shared__ int sched_lds[1024 + 1 + C::NT / 64 + 1];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  using AL = DirectRows<C, C::BM, SrcA, MxArgs, true>;
  using BL = DirectRows<C, C::BN, SrcB, MxArgs, true>;
  constexpr int PERK = AL::PER + BL::PER + 1;             // data loads + one scale load per wave

  RowGroups<C::BM, C::BN, C::NT, ROWS_ALL, C::BM, GROUP_M> sched;
  sched.init(p.offsets, p.E, N, K / 2, sched_lds, sched_lds + 1025);   // K in 16-bit words
  XcdWalk walk;
  walk.init(sched.total);
  if (!walk.valid()) return;
  Tile tl = sched.tile(walk.t);
  MxFragAddr<C> fa;
  fa.init(wm, wn, lane);
  AL al;
  BL bl;
  MxScaleRows<SrcA, SrcB> sc;
  auto init_loaders = [&]() {
    al.init(p, tl);
    bl.init(p, tl);
    sc.init(p, tl, wave);
  };
  auto issue_scales = [&](int kt, int st) { sc.issue(kt, &sscale[st][wave < 4 ? 0 : C::BM], wave); };
  init_loaders();
  int nk = (tl.k_hi - tl.k_lo) / C::BK;
  al.issue(p, tl, 0, smem);
  bl.issue(p, tl, 0, smem + C::A_SLOTS);
  issue_scales(0, 0);
  // The last k step of a tile issues the next tile's first k-tile into the other stage, the
  // epilogue waits for it (one k step old) before its output stores and uses the stage just
  // read as scratch, and the next tile's first k step needs no wait: the output stores drain
  // under that step instead of stalling every workgroup at the tile boundary.
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
      const int cs = (base + kt) & 1, ns = cs ^ 1;
      uint4* st = smem + ns * C::STAGE;
      const int k0 = (kt + 1) * C::BK;
      auto issue = [&](int j) {
        if (j < AL::PER) al.issue_one(p, cur_tile, k0, st, j);
        else if (j < AL::PER + BL::PER) bl.issue_one(p, cur_tile, k0, st + C::A_SLOTS, j - AL::PER);
        else issue_scales(kt + 1, ns);
      };
      mma_ktile_mx<C, true, PERK>(reinterpret_cast<const uint8_t*>(smem + cs * C::STAGE), &sscale[cs][0],
                                  &sscale[cs][C::BM], fa, acc, lane, issue);
    }
    // last k step: its loads are the next tile's first k-tile (without a next tile, this
    // tile's first k-tile again: in bounds, never read, and waited for before the exit)
    if (nk > 1 || !prewaited) wait_vmcnt<0>();
    __syncthreads();
    const int scratch = (base + nk - 1) & 1, ns = scratch ^ 1;
    walk.next();
    const bool more = walk.valid();
    tl = more ? sched.tile(walk.t) : cur_tile;
    init_loaders();
    {
      uint4* st = smem + ns * C::STAGE;
      auto issue = [&](int j) {
        if (j < AL::PER) al.issue_one(p, tl, 0, st, j);
        else if (j < AL::PER + BL::PER) bl.issue_one(p, tl, 0, st + C::A_SLOTS, j - AL::PER);
        else issue_scales(0, ns);
      };
      mma_ktile_mx<C, true, PERK>(reinterpret_cast<const uint8_t*>(smem + scratch * C::STAGE), &sscale[scratch][0],
                                  &sscale[scratch][C::BM], fa, acc, lane, issue);
    }
    // every wave is past its last LDS read before the stage it read becomes scratch
    __syncthreads();
    wait_vmcnt<0>();
    uint8_t* wave_lds = reinterpret_cast<uint8_t*>(smem + scratch * C::STAGE) + wave * RowEpiLds<C>::BYTES;
    Epi::apply(p, cur_tile, acc, wm, wn, lane, wave_lds);
    if (!more) break;
    // the scratch stage receives the next tile's second k-tile: all waves must be done with it
    __syncthreads();
    base = ns;
    nk = (tl.k_hi - tl.k_lo) / C::BK;
    prewaited = true;
  }
}

template <class C, int ACTK = ACT_SWIGLU>
struct MxSwiGLUEpi {  // h = bf16(f(G, U)) -> Hrows (columns as in the bf16 gate/up GEMM)
  __device__ static void apply(const MxArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                               int lane, uint8_t* wlds) {
    stage_store_bf16<C, C::FN * 16, 2>(
        wlds, p.Hrows, p.I, t.m0 + wm * C::WTM, t.m_end, t.nt * (C::BN / 2) + wn * C::FN * 16, p.I, lane,
        [&](int fm, int fn, int q, int j) {
          return gated_act(acc[fm][fn][4 * q + j], acc[fm][fn][4 * q + 8 + j], act_code(ACTK, p.act), p.act_limit);
        },
        [](int fn, int q) { return fn * 16 + q * 8; });
  }
};

template <class C>
struct MxRelu2Epi {  // h = bf16(max(U, 0)^2) -> Hrows (the ungated expert)
  __device__ static void apply(const MxArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                               int lane, uint8_t* wlds) {
    stage_store_bf16<C, C::WTN, 4>(
        wlds, p.Hrows, p.I, t.m0 + wm * C::WTM, t.m_end, t.n0 + wn * C::WTN, p.I, lane,
        [&](int fm, int fn, int q, int j) { return relu2(acc[fm][fn][4 * q + j]); },
        [](int fn, int q) { return fn * 32 + q * 8; });
  }
};

template <class C>
struct MxStoreOEpi {  // O = bf16(acc) -> Orows (streamed past L2 when the host sets stream_out)
  __device__ static void apply(const MxArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                               int lane, uint8_t* wlds) {
    auto val = [&](int fm, int fn, int q, int j) { return acc[fm][fn][4 * q + j]; };
    auto col = [](int fn, int q) { return fn * 32 + q * 8; };
    if (p.stream_out)
      stage_store_bf16<C, C::WTN, 4, true>(wlds, p.Orows, p.H, t.m0 + wm * C::WTM, t.m_end, t.n0 + wn * C::WTN,
                                           p.H, lane, val, col);
    else
      stage_store_bf16<C, C::WTN, 4>(wlds, p.Orows, p.H, t.m0 + wm * C::WTM, t.m_end, t.n0 + wn * C::WTN, p.H,
                                     lane, val, col);
  }
};

__global__ void __launch_bounds__(CfgMx::NT) k_mx_gateup(const MxArgs p) {
  mx_rows_body<CfgMx, MxSrcX, MxSrcGateUpW<CfgMx>, MxSwiGLUEpi<CfgMx>>(p, 2 * p.I, p.H);
}
// any other gated activation (run-time code)
__global__ void __launch_bounds__(CfgMx::NT) k_mx_gateup_act(const MxArgs p) {
  mx_rows_body<CfgMx, MxSrcX, MxSrcGateUpW<CfgMx>, MxSwiGLUEpi<CfgMx, ACT_ANY>>(p, 2 * p.I, p.H);
}
// the ungated ReLU^2 expert (W_up only)
__global__ void __launch_bounds__(CfgMx::NT) k_mx_up(const MxArgs p) {
  mx_rows_body<CfgMx, MxSrcX, MxSrcUpW, MxRelu2Epi<CfgMx>>(p, p.I, p.H);
}
__global__ void __launch_bounds__(CfgMx::NT) k_mx_down(const MxArgs p) {
  // K = I is short: m-tile groups keep the row blocks in L2 while the weight columns stream
  mx_rows_body<CfgMx, MxSrcH, MxSrcDownW, MxStoreOEpi<CfgMx>, 8>(p, p.H, p.I);
}

static int mx_grid(const MxArgs& a, int N) {
  long A = (long)a.T * a.k;
  long mt = A / CfgMx::BM + (a.E < A ? a.E : A) + 1;
  long tiles = mt * ((N + CfgMx::BN - 1) / CfgMx::BN);
  long cap = (long)num_cus();            // one ~136 KB-LDS block per CU
  long g = tiles < cap ? tiles : cap;
  return (int)((g + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
}

hipError_t launch_mx_gateup(const MxArgs& a, hipStream_t s) {
  if (a.act == ACT_RELU2) {
    hipLaunchKernelGGL(k_mx_up, dim3(mx_grid(a, a.I)), dim3(CfgMx::NT), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(a.act == ACT_SWIGLU ? k_mx_gateup : k_mx_gateup_act, dim3(mx_grid(a, 2 * a.I)), dim3(CfgMx::NT),
                     0, s, a);
  return hipGetLastError();
}
hipError_t launch_mx_down(const MxArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_mx_down, dim3(mx_grid(a, a.H)), dim3(CfgMx::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
