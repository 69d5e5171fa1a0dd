// bf16 grouped GEMMs of the MoE layer: forward gate/up + gated activation, forward down,
// and the three row-grouped GEMMs of the backward (direct-to-LDS rows, gemm_rows.h).
#include "gemm_rows.h"
#include "grouped_gemm.h"
#include "kernels.h"

namespace moe {

#ifndef MOE_ROWS_WAVES_N
#define MOE_ROWS_WAVES_N 4
#endif
#ifndef MOE_ROWS_BK
#define MOE_ROWS_BK 64
#endif
// row-grouped GEMMs: 256 x 256 tiles, direct-to-LDS loads, 128 KB of LDS stages
using CfgRows = RowCfg<256, 256, 2, MOE_ROWS_WAVES_N, MOE_ROWS_BK, (MOE_ROWS_BK == 32 ? 4 : 2)>;
// Remainder tiles (the rows of an expert past its last full 256-row block), one per expert
// and GEMM column tile, of the smallest height of 64, 128 or 192 rows that holds them: an
// expert with a few hundred rows streams each weight tile once, with at most 63 rows of
// padding in its MFMAs.
//   192 x 256: two 56 KB stages;  128 x 256: three 48 KB stages;
//   64 x 256:  8 waves side by side, three 40 KB stages.
// the same full tiles on the deep-B schedule (its epilogue stages 4 KB per wave in one A stage)
using CfgRowsDB = RowCfg<256, 256, 2, 4, 64, 2, 4096>;
using CfgRem192 = RowCfg<192, 256, 2, 4, 64, 2>;
using CfgRem128 = RowCfg<128, 256, 2, 4, 64, 3>;
using CfgRem64 = RowCfg<64, 256, 1, 8, 64, 3>;
// the ungated (ReLU^2) recompute: 128 x 256 tiles, three 48 KB stages (its epilogue, with
// 256-row tiles, would spill)
using CfgRecUp = RowCfg<128, 256, 2, 4, 64, 3>;

// ------------------------------------------------------------------------
// Row sources of the direct-to-LDS row-grouped GEMMs: a wave-uniform base and
// a 32-bit element offset per row; rows past the expert's segment (columns past
// N) are clamped to a valid one and their results are never stored.
// ------------------------------------------------------------------------
__device__ __forceinline__ int clamp_row(const Tile& t, int row) { return min(t.m0 + row, t.m_end - 1); }

struct RSrcX {
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile&, int, int k0) { return p.X + k0; }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    return (uint32_t)p.row_token[clamp_row(t, row)] * (uint32_t)p.H;
  }
};
struct RSrcDY {
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile&, int, int k0) { return p.dY + k0; }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    return (uint32_t)p.row_token[clamp_row(t, row)] * (uint32_t)p.H;
  }
};
struct RSrcH {
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile&, int, int k0) { return p.Hrows + k0; }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    return (uint32_t)clamp_row(t, row) * (uint32_t)p.I;
  }
};
struct RSrcDGU {
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile&, int, int k0) { return p.dGU + k0; }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    return (uint32_t)clamp_row(t, row) * (uint32_t)(2 * p.I);
  }
};
// Packed gate / up weights [E, I, H].  Inside every 32-row MFMA fragment of the
// B tile, rows 0-15 are gate columns and rows 16-31 the up columns of the same
// 16 intermediate indices, so an accumulator lane holds each (gate, up) pair
// at items v and v + 8 of one fragment.
template <class C>
struct RSrcGateUpW {
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile& t, int row0, int k0) {
    const bool up = (row0 % 32) >= 16;
    return (up ? p.Wu_t : p.Wg_t) + (size_t)t.e * p.I * p.H + k0;
  }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    const int col = t.nt * (C::BN / 2) + (row / 32) * 16 + (row % 16);
    return (uint32_t)min(col, p.I - 1) * (uint32_t)p.H;
  }
};
struct RSrcUpW {         // packed W_up [E, I, H]: the B rows of the ungated (ReLU^2) up GEMM
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile& t, int, int k0) {
    return p.Wu_t + (size_t)t.e * p.I * p.H + k0;
  }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    return (uint32_t)min(t.n0 + row, p.I - 1) * (uint32_t)p.H;
  }
};
// du rows of the ungated backward as [T*k, K = 2I]: the bf16 values [T*k, I] then their bf16
// remainders [T*k, I]
struct RSrcDU2 {
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile&, int, int k0) {
    return k0 < p.I ? p.dGU + k0 : p.dGU_lo + (k0 - p.I);
  }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    return (uint32_t)clamp_row(t, row) * (uint32_t)p.I;
  }
};
struct RSrcDownW {       // packed [E, H, I]
  __device__ static const uint16_t* base(const GemmArgs& p, const Tile& t, int, int k0) {
    return p.Wd_t + (size_t)t.e * p.H * p.I + k0;
  }
  __device__ static uint32_t row_off(const GemmArgs& p, const Tile& t, int row) {
    return (uint32_t)min(t.n0 + row, p.H - 1) * (uint32_t)p.I;
  }
};
// k-major B sources of the backward's row GEMMs: the packed weights (the forward's layout)
// read transposed, so the backward needs no math-layout copy (KMajorRowsB).
struct KSrcDownWt {      // W_down^T: Wd_t [E, H, I] as [K = H, N = I]
  __device__ static const uint16_t* kbase(const GemmArgs& p, const Tile& t, int k0) {
    return p.Wd_t + (size_t)t.e * p.H * p.I + (size_t)k0 * p.I;
  }
  __device__ static int ld(const GemmArgs& p) { return p.I; }
  __device__ static int ncols(const GemmArgs& p) { return p.I; }
};
struct KSrcGateUpWt {    // [W_gate | W_up]^T: [Wg_t | Wu_t] [E, I, H] as [K = 2I, N = H]
  __device__ static const uint16_t* kbase(const GemmArgs& p, const Tile& t, int k0) {
    const size_t e0 = (size_t)t.e * p.I * p.H;
    return k0 < p.I ? p.Wg_t + e0 + (size_t)k0 * p.H : p.Wu_t + e0 + (size_t)(k0 - p.I) * p.H;
  }
  __device__ static int ld(const GemmArgs& p) { return p.H; }
  __device__ static int ncols(const GemmArgs& p) { return p.H; }
};
struct KSrcUpWt2 {       // W_up^T twice along K: Wu_t [E, I, H] as [K = 2I, N = H] (ReLU^2 dX)
  __device__ static const uint16_t* kbase(const GemmArgs& p, const Tile& t, int k0) {
    return p.Wu_t + (size_t)t.e * p.I * p.H + (size_t)(k0 < p.I ? k0 : k0 - p.I) * p.H;
  }
  __device__ static int ld(const GemmArgs& p) { return p.H; }
  __device__ static int ncols(const GemmArgs& p) { return p.H; }
};

// ------------------------------------------------------------------------
// Ops: schedule + loaders + epilogue of each GEMM
// ------------------------------------------------------------------------
// PART: which rows of each expert the schedule covers (all of them, its full 256-row blocks,
// or one of the three remainder classes; RowPart).
template <class C, class SrcA_, class SrcB_, int PART = ROWS_ALL>
struct RowOpsBase {
  using SrcA = SrcA_;
  using SrcB = SrcB_;
  using Sched = RowGroups<C::BM, C::BN, C::NT, PART, (PART == ROWS_ALL ? C::BM : 256)>;
};

// Saved-activation forward: the fp32 projections of the tile's valid rows into GU [A, 2I] (G in
// columns [0, I), U in [I, 2I)), straight from the accumulators: 16 bytes per lane, 32
// contiguous bytes per row from the two lane halves (plain stores: as non-temporal stores these
// partial-line writes made the training forward's gate/up GEMM 1,239 -> 1,464 us).  Item group q
// of fragment fn holds columns col_of(fn, q) + 4 (lane / 32) + [0, 4) (relative to c0); gate(q) /
// up(q) name its accumulator items (-1: none).
template <class C, int NQ, class Col, class Gate, class Up>
__device__ __forceinline__ void store_gu_f32(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm,
                                             int c0, int lane, Col col_of, Gate gate, Up up) {
  const int hc = (lane >> 5) * 4;
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int r = t.m0 + Frag<C>::row(wm, fm, lane);
    if (r >= t.m_end) continue;
    float* row = p.GU + (size_t)r * (2 * p.I);
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int c = c0 + col_of(fn, q) + hc;
        if (c >= p.I) continue;
        if (gate(q) >= 0) {
          const int v = gate(q);
          *reinterpret_cast<float4*>(row + c) =
              make_float4(acc[fm][fn][v], acc[fm][fn][v + 1], acc[fm][fn][v + 2], acc[fm][fn][v + 3]);
        }
        if (up(q) >= 0) {
          const int v = up(q);
          *reinterpret_cast<float4*>(row + p.I + c) =
              make_float4(acc[fm][fn][v], acc[fm][fn][v + 1], acc[fm][fn][v + 2], acc[fm][fn][v + 3]);
        }
      }
  }
}

// h = bf16(f(X Wg, X Wu)), f the problem's gated activation (SwiGLU by default)
template <class C, int PART = ROWS_ALL, int ACTK = ACT_SWIGLU>
struct FwdGateUpOps : RowOpsBase<C, RSrcX, RSrcGateUpW<C>, PART> {
  __device__ static void init_sched(typename RowOpsBase<C, RSrcX, RSrcGateUpW<C>, PART>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, 2 * p.I, p.H, pre, red);
  }
  // the h stores are counted; the saved-activation forward's G, U stores are not
  static constexpr int OUT_STORES = stage_store_count<C, C::FN * 16>();
  __device__ static bool stores_counted(const GemmArgs& p) { return p.GU == nullptr; }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t* wlds) {
    // fragment fn holds intermediate columns (wn * FN + fn) * 16 + [0, 16): items 4q + j (q = 0, 1)
    // are gate and 4q + 8 + j the up values of column 8q + 4 * (lane / 32) + j
    stage_store_bf16<C, C::FN * 16, 2, false, true>(
        wlds, p.Hrows, p.I, t.m0 + wm * C::WTM, t.m_end, t.nt * (C::BN / 2) + wn * C::FN * 16, p.I, lane,
        [&](int fm, int fn, int q, int j) {
          return gated_act(acc[fm][fn][4 * q + j], acc[fm][fn][4 * q + 8 + j], act_code(ACTK, p.act), p.act_limit);
        },
        [](int fn, int q) { return fn * 16 + q * 8; });
    if (p.GU)
      store_gu_f32<C, 2>(
          p, t, acc, wm, t.nt * (C::BN / 2) + wn * C::FN * 16, lane, [](int fn, int q) { return fn * 16 + q * 8; },
          [](int q) { return 4 * q; }, [](int q) { return 4 * q + 8; });
  }
};

// h = bf16(max(X Wu, 0)^2): the ungated (ReLU^2) expert, one GEMM over the I columns
template <class C, int PART = ROWS_ALL>
struct FwdUpOps : RowOpsBase<C, RSrcX, RSrcUpW, PART> {
  __device__ static void init_sched(typename RowOpsBase<C, RSrcX, RSrcUpW, PART>::Sched& s, const GemmArgs& p,
                                    int* pre, int* red) {
    s.init(p.offsets, p.E, p.I, p.H, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t* wlds) {
    stage_store_bf16<C, C::WTN, 4>(
        wlds, p.Hrows, p.I, t.m0 + wm * C::WTM, t.m_end, t.n0 + wn * C::WTN, p.I, lane,
        [&](int fm, int fn, int q, int j) { return relu2(acc[fm][fn][4 * q + j]); },
        [](int fn, int q) { return fn * 32 + q * 8; });
    if (p.GU)
      store_gu_f32<C, 4>(
          p, t, acc, wm, t.n0 + wn * C::WTN, lane, [](int fn, int q) { return fn * 32 + q * 8; },
          [](int) { return -1; }, [](int q) { return 4 * q; });
  }
};

// fp32 rows straight from the accumulators: each lane writes its 16-byte item
// groups (32 contiguous bytes per row from the two lane halves).  Every wave issues exactly
// FM * FN * 4 buffer stores (rows at or past the segment's end and columns at or past ncols
// dropped by the resource's range), the count the deep-B schedule waits on.
template <class C>
__device__ __forceinline__ void store_rows_f32(float* base, int ld, int ncols, const Tile& t,
                                               f32x16 (&acc)[C::FM][C::FN], int wm, int wn, int lane) {
  const int row0 = t.m0 + wm * C::WTM;                   // the wave's first row
  const int valid = min(max(t.m_end - row0, 0), C::WTM);
  const __amdgpu_buffer_rsrc_t rs = out_rsrc(base + (size_t)row0 * ld, (uint32_t)valid * (uint32_t)ld * 4u);
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const uint32_t rrel = (uint32_t)(fm * 32 + (lane & 31));
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = t.n0 + Frag<C>::col(wn, fn, q, lane);
        const uint32_t off = n < ncols ? (rrel * (uint32_t)ld + (uint32_t)n) * 4u : BUF_DROP;
        buf_store16(rs, off, __float_as_uint(acc[fm][fn][4 * q]), __float_as_uint(acc[fm][fn][4 * q + 1]),
                    __float_as_uint(acc[fm][fn][4 * q + 2]), __float_as_uint(acc[fm][fn][4 * q + 3]));
      }
  }
}
template <class C>
constexpr int store_rows_f32_count() { return C::FM * C::FN * 4; }

// O = bf16(h Wd)
template <class C, int PART = ROWS_ALL>
struct FwdDownOps : RowOpsBase<C, RSrcH, RSrcDownW, PART> {
  __device__ static void init_sched(typename RowOpsBase<C, RSrcH, RSrcDownW, PART>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, p.H, p.I, pre, red);
  }
  static constexpr int OUT_STORES = stage_store_count<C, C::WTN>();
  __device__ static bool stores_counted(const GemmArgs&) { return true; }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t* wlds) {
    stage_store_bf16<C, C::WTN, 4, false, true>(
        wlds, p.Orows, p.H, t.m0 + wm * C::WTM, t.m_end, t.n0 + wn * C::WTN, p.H, lane,
        [&](int fm, int fn, int q, int j) { return acc[fm][fn][4 * q + j]; },
        [](int fn, int q) { return fn * 32 + q * 8; });
  }
};

// P = dY[token] W_down^T (fp32), W_down^T read from the packed Wd_t
template <class C, int PART = ROWS_ALL>
struct BwdPOps : RowOpsBase<C, RSrcDY, KSrcDownWt, PART> {
  static constexpr bool B_KMAJOR = true;
  __device__ static void init_sched(typename RowOpsBase<C, RSrcDY, KSrcDownWt, PART>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, p.I, p.H, pre, red);
  }
  static constexpr int OUT_STORES = store_rows_f32_count<C>();
  __device__ static bool stores_counted(const GemmArgs&) { return true; }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t*) {
    store_rows_f32<C>(p.P, p.I, p.I, t, acc, wm, wn, lane);
  }
};

// v = hi + lo with hi = bf16(v), lo = bf16(v - hi), four values packed in pairs.
__device__ __forceinline__ void split4(const float (&v)[4], uint2& hi, uint2& lo) {
  hi.x = pack_bf16x2(v[0], v[1]);
  hi.y = pack_bf16x2(v[2], v[3]);
  lo.x = pack_bf16x2(v[0] - bf16_to_f32(hi.x & 0xffffu), v[1] - bf16_to_f32(hi.x >> 16));
  lo.y = pack_bf16x2(v[2] - bf16_to_f32(hi.y & 0xffffu), v[3] - bf16_to_f32(hi.y >> 16));
}

// Recompute G, U; with P give the router-weight partial sums <h, P> (h = bf16(f(G, U)))
// and the operands of the weight gradients: w h, dg and du, each as a bf16 value and a
// bf16 remainder.  A wave owns 32 intermediate columns of WTM rows.  P is read one 32-row
// block ahead of its use; the six bf16 outputs of each 32-row block go through the wave's
// LDS scratch (four staged blocks, then two) and leave as whole 64-byte row segments
// (16 bytes per lane).  du is recomputed from the accumulators for the second round
// rather than held in registers.
template <class C, int PART = ROWS_ALL, int ACTK = ACT_SWIGLU>
struct BwdRecomputeOps : RowOpsBase<C, RSrcX, RSrcGateUpW<C>, PART> {
  __device__ static void init_sched(typename RowOpsBase<C, RSrcX, RSrcGateUpW<C>, PART>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, 2 * p.I, p.H, pre, red);
  }
  // its epilogue runs at the register limit: the plain two-stage schedule
  static constexpr bool EARLY_NEXT = false;
  // one staged 32 x 32 bf16 block: 64-byte rows, 16-byte chunk c of row r at c ^ ((r >> 2) & 3)
  static constexpr int OUT = 32 * 64;
  // three rounds of two staged blocks (w h, dg, du each computed from the accumulators) for the
  // run-time activation, whose switch needs the registers, and for tiles whose LDS scratch holds
  // two blocks only; else two rounds (four blocks, then two)
  static constexpr bool THREE_ROUNDS = ACTK == ACT_ANY || RowEpiLds<C>::BYTES < 4 * OUT;
  static_assert(C::FN * 16 == 32, "a wave owns 32 intermediate columns");
  static_assert(RowEpiLds<C>::BYTES >= (THREE_ROUNDS ? 2 : 4) * OUT, "staging area too small");

  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t* wlds) {
    const int col0 = t.nt * (C::BN / 2) + wn * 32;   // first intermediate column of the wave
    const bool cv = col0 < p.I;                       // I is a multiple of 32: all or none valid
    const int h = lane >> 5;
    // P and the row weight of row block fm (rows past the segment read a valid row),
    // one block ahead of its use
    float4 P4[2][C::FN][2];
    float wr[2];
    auto load_p = [&](int fm, int buf) {
      const int r = min(t.m0 + Frag<C>::row(wm, fm, lane), t.m_end - 1);
      wr[buf] = p.topk_w[p.row_slot[r]];
      const float* Prow = p.P + (size_t)r * p.I + col0 + h * 4;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          P4[buf][fn][q] = cv ? *reinterpret_cast<const float4*>(Prow + fn * 16 + q * 8) : make_float4(0, 0, 0, 0);
    };
    load_p(0, 0);
    // same (gate, up) pairing as the forward: items 4q + j and 4q + 8 + j of fragment fn
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      if (fm + 1 < C::FM) load_p(fm + 1, (fm + 1) & 1);
      const int r = t.m0 + Frag<C>::row(wm, fm, lane);
      const float w = wr[fm & 1];
      float dot = 0.f;
      const int rl = lane & 31;
      // chunk (2 fn + q) of staged block o, this lane's row and half
      auto slot = [&](int o, int fn, int q) {
        return reinterpret_cast<uint2*>(wlds + o * OUT + rl * 64 + (((2 * fn + q) ^ ((rl >> 2) & 3)) * 16) + h * 8);
      };
      const int act = act_code(ACTK, p.act);
      const int row0 = t.m0 + wm * C::WTM + fm * 32;
      // output o: 0 w h, 1 its remainder, 2 dg, 3 its remainder, 4 du, 5 its remainder
      auto flush = [&](int s, int o) {
        uint16_t* out = o == 0 ? p.hw : o == 1 ? p.hw_lo : (o & 1) ? p.dGU_lo + (o == 5 ? p.I : 0)
                                                                    : p.dGU + (o == 4 ? p.I : 0);
        const int ld = o < 2 ? p.I : 2 * p.I;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int idx = i * 64 + lane, rr = idx >> 2, ch = idx & 3;
          const uint4 v = *reinterpret_cast<const uint4*>(wlds + s * OUT + rr * 64 + ((ch ^ ((rr >> 2) & 3)) * 16));
          if (row0 + rr < t.m_end) *reinterpret_cast<uint4*>(out + (size_t)(row0 + rr) * ld + col0 + ch * 8) = v;
        }
      };
      if constexpr (THREE_ROUNDS) {
        // three rounds of two slots, each computing one quantity from the accumulators -- w h
        // with the partial sum, dg, du
#pragma unroll
        for (int o = 0; o < 6; o += 2) {
#pragma unroll
          for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const float4 pv = P4[fm & 1][fn][q];
              const float Pv[4] = {pv.x, pv.y, pv.z, pv.w};
              float v[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const float g = acc[fm][fn][4 * q + j], u = acc[fm][fn][4 * q + 8 + j];
                if (o == 0) {
                  const float hv = bf16_to_f32(f32_to_bf16(gated_act(g, u, act, p.act_limit)));
                  dot += hv * Pv[j];
                  v[j] = w * hv;
                } else {
                  v[j] = w * Pv[j] * (o == 2 ? gated_act_dg(g, u, act, p.act_limit)
                                             : gated_act_du(g, u, act, p.act_limit));
                }
              }
              uint2 hi, lo;
              split4(v, hi, lo);
              *slot(0, fn, q) = hi;
              *slot(1, fn, q) = lo;
            }
          if (o == 0) {
            // the other half of this row's columns sits in lane ^ 32
            dot += __shfl_xor(dot, 32, 64);
            if (r < t.m_end && lane < 32) p.dwt_part[(size_t)r * p.nparts + t.nt * C::WAVES_N + wn] = dot;
          }
          if (cv) {
            flush(0, o);
            flush(1, o + 1);
          }
        }
        continue;
      }
      // round 1: w h and dg (values and remainders) into slots 0..3, and the partial sum
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float4 pv = P4[fm & 1][fn][q];
          const float Pv[4] = {pv.x, pv.y, pv.z, pv.w};
          float hw[4], dg[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float hf, fg, fu;
            gated_act_grad(acc[fm][fn][4 * q + j], acc[fm][fn][4 * q + 8 + j], act, p.act_limit, hf, fg, fu);
            const float hv = bf16_to_f32(f32_to_bf16(hf));
            dot += hv * Pv[j];
            hw[j] = w * hv;
            dg[j] = w * Pv[j] * fg;
          }
          if (cv) {
            uint2 hi, lo;
            split4(hw, hi, lo);
            *slot(0, fn, q) = hi;
            *slot(1, fn, q) = lo;
            split4(dg, hi, lo);
            *slot(2, fn, q) = hi;
            *slot(3, fn, q) = lo;
          }
        }
      // the other half of this row's columns sits in lane ^ 32
      dot += __shfl_xor(dot, 32, 64);
      if (r < t.m_end && lane < 32) p.dwt_part[(size_t)r * p.nparts + t.nt * C::WAVES_N + wn] = dot;
      if (!cv) continue;
#pragma unroll
      for (int o = 0; o < 4; ++o) flush(o, o);
      // round 2: du (value and remainder) into slots 0..1 (a wave's LDS operations keep their order)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float4 pv = P4[fm & 1][fn][q];
          const float Pv[4] = {pv.x, pv.y, pv.z, pv.w};
          float du[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            du[j] = w * Pv[j] * gated_act_du(acc[fm][fn][4 * q + j], acc[fm][fn][4 * q + 8 + j], act, p.act_limit);
          uint2 hi, lo;
          split4(du, hi, lo);
          *slot(0, fn, q) = hi;
          *slot(1, fn, q) = lo;
        }
      flush(0, 4);
      flush(1, 5);
    }
  }
};

// The ungated (ReLU^2) recompute: U again; with P give, for h = bf16(max(U, 0)^2), the
// router-weight partial sums <h, P>, w h and du = w P 2 max(U, 0), each as a bf16 value and a
// bf16 remainder.  A wave owns 64 columns.  The three bf16 outputs are staged through the wave's
// LDS scratch one after another, each computed from U and P as it goes (P is read once per
// output: holding it across them would spill).
template <class C, int PART = ROWS_ALL>
struct BwdRecomputeUpOps : RowOpsBase<C, RSrcX, RSrcUpW, PART> {
  __device__ static void init_sched(typename RowOpsBase<C, RSrcX, RSrcUpW, PART>::Sched& s, const GemmArgs& p,
                                    int* pre, int* red) {
    s.init(p.offsets, p.E, p.I, p.H, pre, red);
  }

  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t* wlds) {
    const int col0 = t.n0 + wn * C::WTN;            // first intermediate column of the wave
    const bool cv = col0 < p.I;                      // I is a multiple of 64: all or none valid
    const int hc = (lane >> 5) * 4;
    auto row_of = [&](int fm) { return min(t.m0 + Frag<C>::row(wm, fm, lane), t.m_end - 1); };
    // P of item group q of fragment (fm, fn) (zeros for columns past I)
    auto p4 = [&](int rc, int fn, int q) {
      return cv ? *reinterpret_cast<const float4*>(p.P + (size_t)rc * p.I + col0 + fn * 32 + q * 8 + hc)
                : make_float4(0, 0, 0, 0);
    };
    // router-weight partial sums: <bf16(h), P> over the wave's columns of each row
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int rc = row_of(fm);
      float dot = 0.f;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 pv = p4(rc, fn, q);
          const float Pv[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) dot += bf16_to_f32(f32_to_bf16(relu2(acc[fm][fn][4 * q + j]))) * Pv[j];
        }
      dot += __shfl_xor(dot, 32, 64);                // the other half of the row's columns
      const int r = t.m0 + Frag<C>::row(wm, fm, lane);
      if (r < t.m_end && lane < 32) p.dwt_part[(size_t)r * p.nparts + t.nt * C::WAVES_N + wn] = dot;
    }
    if (!cv) return;
    const int row0 = t.m0 + wm * C::WTM;
    auto col_of = [](int fn, int q) { return fn * 32 + q * 8; };
    // w h with h = bf16(max(U, 0)^2), as a bf16 value and a bf16 remainder
    auto hw = [&](int fm, int fn, int q, int j) {
      return p.topk_w[p.row_slot[row_of(fm)]] * bf16_to_f32(f32_to_bf16(relu2(acc[fm][fn][4 * q + j])));
    };
    stage_store_bf16<C, C::WTN, 4>(wlds, p.hw, p.I, row0, t.m_end, col0, p.I, lane, hw, col_of);
    stage_store_bf16<C, C::WTN, 4>(
        wlds, p.hw_lo, p.I, row0, t.m_end, col0, p.I, lane,
        [&](int fm, int fn, int q, int j) {
          const float v = hw(fm, fn, q, j);
          return v - bf16_to_f32(f32_to_bf16(v));
        },
        col_of);
    // du for item j of group q: w P 2 max(U, 0)
    auto du = [&](int fm, int fn, int q, int j) {
      const int rc = row_of(fm);
      const float Pj = p.P[(size_t)rc * p.I + col0 + fn * 32 + q * 8 + hc + j];
      return p.topk_w[p.row_slot[rc]] * Pj * relu2_grad(acc[fm][fn][4 * q + j]);
    };
    stage_store_bf16<C, C::WTN, 4>(wlds, p.dGU, p.I, row0, t.m_end, col0, p.I, lane, du, col_of);
    stage_store_bf16<C, C::WTN, 4>(
        wlds, p.dGU_lo, p.I, row0, t.m_end, col0, p.I, lane,
        [&](int fm, int fn, int q, int j) {
          const float v = du(fm, fn, q, j);
          return v - bf16_to_f32(f32_to_bf16(v));
        },
        col_of);
  }
};

// dXr = du W_up^T (fp32 rows) of the ungated expert, with du as its bf16 value plus its bf16
// remainder (two passes over I): ReLU^2's du = w P 2 max(U, 0) reaches several units, and
// its bf16 value alone leaves dX short of the exact-du result near cancellations
template <class C, int PART = ROWS_ALL>
struct BwdDXUpOps : RowOpsBase<C, RSrcDU2, KSrcUpWt2, PART> {
  static constexpr bool B_KMAJOR = true;
  __device__ static void init_sched(typename RowOpsBase<C, RSrcDU2, KSrcUpWt2, PART>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, p.H, 2 * p.I, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t*) {
    store_rows_f32<C>(p.dXr, p.H, p.H, t, acc, wm, wn, lane);
  }
};

// dXr = [dg | du] [W_gate | W_up]^T (fp32 rows), the weights read from the packed Wg_t, Wu_t
template <class C, int PART = ROWS_ALL>
struct BwdDXOps : RowOpsBase<C, RSrcDGU, KSrcGateUpWt, PART> {
  static constexpr bool B_KMAJOR = true;
  static constexpr int OUT_STORES = store_rows_f32_count<C>();
  __device__ static bool stores_counted(const GemmArgs&) { return true; }
  __device__ static void init_sched(typename RowOpsBase<C, RSrcDGU, KSrcGateUpWt, PART>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, p.H, 2 * p.I, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane, uint8_t*) {
    store_rows_f32<C>(p.dXr, p.H, p.H, t, acc, wm, wn, lane);
  }
};

// ------------------------------------------------------------------------
// Kernels and launchers
// ------------------------------------------------------------------------
#define MOE_ROWS_SPLIT_KERNEL(NAME, OPS)                                                            \
  __global__ void __launch_bounds__(CfgRows::NT) NAME(const GemmArgs p) {                            \
    rows_gemm_split_body<CfgRows, CfgRem192, CfgRem128, CfgRem64, OPS<CfgRows, ROWS_FULL>,           \
                         OPS<CfgRem192, ROWS_REM_Q3>, OPS<CfgRem128, ROWS_REM_Q2>,                   \
                         OPS<CfgRem64, ROWS_REM_Q1>, GemmArgs>(p);                                    \
  }

// the gated activation as a run-time code (every activation but the default SwiGLU)
template <class C, int PART>
using FwdGateUpOpsAny = FwdGateUpOps<C, PART, ACT_ANY>;
template <class C>
using BwdRecomputeOpsAny = BwdRecomputeOps<C, ROWS_ALL, ACT_ANY>;
// the gated recompute with a run-time activation: 128 x 256 tiles, three 48 KB stages (its
// activation switch does not fit the registers of 256-row tiles)
using CfgRecAny = RowCfg<128, 256, 2, 4, 64, 3>;

// the four passes, the full one on the deep-B schedule
#define MOE_ROWS_SPLIT_DB_KERNEL(NAME, OPS)                                                         \
  __global__ void __launch_bounds__(CfgRowsDB::NT) NAME(const GemmArgs p) {                          \
    rows_gemm_split_body_db<CfgRowsDB, CfgRem192, CfgRem128, CfgRem64, OPS<CfgRowsDB, ROWS_FULL>,    \
                            OPS<CfgRem192, ROWS_REM_Q3>, OPS<CfgRem128, ROWS_REM_Q2>,                \
                            OPS<CfgRem64, ROWS_REM_Q1>, GemmArgs>(p);                                \
  }
MOE_ROWS_SPLIT_DB_KERNEL(k_fwd_gateup, FwdGateUpOps)
MOE_ROWS_SPLIT_DB_KERNEL(k_fwd_gateup_act, FwdGateUpOpsAny)
MOE_ROWS_SPLIT_DB_KERNEL(k_fwd_down, FwdDownOps)
MOE_ROWS_SPLIT_DB_KERNEL(k_bwd_p, BwdPOps)
// the recompute over the four row passes: the remainders of at most 64 rows take 64 x 256 tiles
// of 8 waves of 32 x 64 (every pass keeps 4 waves across the 256 columns, as the router-weight
// partial sums are laid out)
using CfgRecRem64 = RowCfg<64, 256, 2, 4, 64, 3>;
__global__ void __launch_bounds__(CfgRows::NT) k_bwd_recompute(const GemmArgs p) {
  rows_gemm_split_body<CfgRows, CfgRem192, CfgRem128, CfgRecRem64, BwdRecomputeOps<CfgRows, ROWS_FULL>,
                       BwdRecomputeOps<CfgRem192, ROWS_REM_Q3>, BwdRecomputeOps<CfgRem128, ROWS_REM_Q2>,
                       BwdRecomputeOps<CfgRecRem64, ROWS_REM_Q1>, GemmArgs>(p);
}
__global__ void __launch_bounds__(CfgRecAny::NT) k_bwd_recompute_act(const GemmArgs p) {
  rows_gemm_body<CfgRecAny, BwdRecomputeOpsAny<CfgRecAny>, GemmArgs>(p);
}
MOE_ROWS_SPLIT_DB_KERNEL(k_bwd_dx_rows, BwdDXOps)
// the ungated (ReLU^2) expert
MOE_ROWS_SPLIT_KERNEL(k_fwd_up, FwdUpOps)
__global__ void __launch_bounds__(CfgRecUp::NT) k_bwd_recompute_up(const GemmArgs p) {
  rows_gemm_body<CfgRecUp, BwdRecomputeUpOps<CfgRecUp>, GemmArgs>(p);
}
MOE_ROWS_SPLIT_KERNEL(k_bwd_dx_rows_up, BwdDXUpOps)

template <class C>
static int row_grid(const GemmArgs& a, int N) {
  long A = (long)a.T * a.k;
  long mt = A / C::BM + (a.E < A ? a.E : A) + 1;
  long tiles = mt * ((N + C::BN - 1) / C::BN);
  long cap = (long)num_cus();            // one block per CU (its LDS stages fill most of the 160 KB)
  long g = tiles < cap ? tiles : cap;
  return (int)((g + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
}
// grid of a kernel on lane tables: every pass's tiles fit 64 per workgroup
static int lane_row_grid(const GemmArgs& a, int N) {
  const long A = (long)a.T * a.k;
  const long bound = (A / 256 + (a.E < A ? a.E : A) + 1) * ((N + 255) / 256);
  return lanes_grid(bound, (long)num_cus());
}
hipError_t launch_fwd_gateup(const GemmArgs& a, hipStream_t s) {
  if (a.act == ACT_RELU2) {
    hipLaunchKernelGGL(k_fwd_up, dim3(row_grid<CfgRows>(a, a.I)), dim3(CfgRows::NT), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(a.act == ACT_SWIGLU ? k_fwd_gateup : k_fwd_gateup_act, dim3(lane_row_grid(a, 2 * a.I)),
                     dim3(CfgRowsDB::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_fwd_down(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_fwd_down, dim3(lane_row_grid(a, a.H)), dim3(CfgRowsDB::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bwd_p(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_p, dim3(lane_row_grid(a, a.I)), dim3(CfgRowsDB::NT), 0, s, a);
  return hipGetLastError();
}
int bwd_nparts(int I, int act) {
  const int N = act_gated(act) ? 2 * I : I;        // columns of the recompute GEMM
  return ((N + CfgRows::BN - 1) / CfgRows::BN) * CfgRows::WAVES_N;
}
hipError_t launch_bwd_recompute(const GemmArgs& a, hipStream_t s) {
  if (a.act == ACT_RELU2) {
    hipLaunchKernelGGL(k_bwd_recompute_up, dim3(row_grid<CfgRecUp>(a, a.I)), dim3(CfgRecUp::NT), 0, s, a);
    return hipGetLastError();
  }
  if (a.act == ACT_SWIGLU)
    hipLaunchKernelGGL(k_bwd_recompute, dim3(row_grid<CfgRows>(a, 2 * a.I)), dim3(CfgRows::NT), 0, s, a);
  else
    hipLaunchKernelGGL(k_bwd_recompute_act, dim3(row_grid<CfgRecAny>(a, 2 * a.I)), dim3(CfgRecAny::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bwd_dx_rows(const GemmArgs& a, hipStream_t s) {
  if (a.act == ACT_RELU2)
    hipLaunchKernelGGL(k_bwd_dx_rows_up, dim3(row_grid<CfgRows>(a, a.H)), dim3(CfgRows::NT), 0, s, a);
  else
    hipLaunchKernelGGL(k_bwd_dx_rows, dim3(lane_row_grid(a, a.H)), dim3(CfgRowsDB::NT), 0, s, a);
  return hipGetLastError();
}
// dX[t] = bf16(sum_j dXr[slot_row[t*k+j]]), d_topk_w[t,j] = sum of the row's partials (slots
// without a row, slot_row < 0, add nothing and get d_topk_w = 0).
// One wave per (token, slice of 64 chunks of 8 fp32): the token's row indices are
// wave-uniform, each lane issues the loads of four rows before it adds them (ascending j).
// The fp32 rows take plain cached loads: part of them, just written by the dX-rows GEMM,
// still sits in the caches (the nontemporal hint measured 10% slower on the training shape).
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4v load_f32x4(const float* ptr) { return *reinterpret_cast<const f32x4v*>(ptr); }
__device__ __forceinline__ void add8(float (&acc)[8], const f32x4v& a, const f32x4v& b) {
  acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
  acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
}

__global__ void __launch_bounds__(256) k_bwd_token_reduce(const GemmArgs p, const int32_t* slot_row,
                                                          uint16_t* dX, float* dtw) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunks = p.H / 8;
  const int slices = (chunks + 63) / 64;
  const long units = (long)p.T * slices;
  for (long u = (long)blockIdx.x * 4 + wave; u < units; u += (long)gridDim.x * 4) {
    const int t = (int)(u / slices), sl = (int)(u - (long)t * slices);
    const int32_t* sr = slot_row + (size_t)t * p.k;
    const int c = sl * 64 + lane;
    const bool has = c < chunks;
    const int cc = has ? c : 0;                     // in-bounds reads for idle lanes
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j = 0;
    for (; j + 4 <= p.k; j += 4) {
      f32x4v v[4][2];
      int rr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rr[q] = sr[j + q];
        const float* src = p.dXr + (size_t)max(rr[q], 0) * p.H + cc * 8;
        v[q][0] = load_f32x4(src);
        v[q][1] = load_f32x4(src + 4);
      }
      __builtin_amdgcn_sched_barrier(0);           // all eight loads in flight before the adds
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (rr[q] >= 0) add8(acc, v[q][0], v[q][1]);
    }
    for (; j < p.k; ++j) {
      const int r = sr[j];
      if (r < 0) continue;
      const float* src = p.dXr + (size_t)r * p.H + cc * 8;
      add8(acc, load_f32x4(src), load_f32x4(src + 4));
    }
    if (has) {
      uint4 o;
      o.x = pack_bf16x2(acc[0], acc[1]);
      o.y = pack_bf16x2(acc[2], acc[3]);
      o.z = pack_bf16x2(acc[4], acc[5]);
      o.w = pack_bf16x2(acc[6], acc[7]);
      *reinterpret_cast<uint4*>(dX + (size_t)t * p.H + c * 8) = o;
    }
    // d_topk_w: lane j of the token's first slice sums slot j's partials (k <= 32 lanes), eight
    // loads in flight (eight running sums added in a fixed order at the end)
    if (sl == 0 && lane < p.k) {
      const int r = sr[lane];
      float s8[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (r >= 0) {
        const float* part = p.dwt_part + (size_t)r * p.nparts;
        int q = 0;
        for (; q + 8 <= p.nparts; q += 8) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = part[q + i];
#pragma unroll
          for (int i = 0; i < 8; ++i) s8[i] += v[i];
        }
        for (; q < p.nparts; ++q) s8[0] += part[q];
      }
      dtw[t * p.k + lane] = ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
    }
  }
}

// Saved-activation backward, in place of the recompute: per expert-major row r (weight
// w = topk_w[row_slot[r]]), from P and the saved fp32 G, U the same quantities the recompute's
// epilogue forms from its accumulators, with the same expressions: h = bf16(f(G, U)),
// <h, P> (one partial sum per row, dwt_part[r]), and w h, dg = w P df/dG, du = w P df/dU,
// each as a bf16 value and a bf16 remainder.  One wave per row, four columns per lane and
// step (16-byte loads, 8-byte stores); the row's partial sum adds the lanes' sums in a fixed
// butterfly.  Rows at or past expert_offsets[E] (slots dispatch skipped) have none of these.
__global__ void __launch_bounds__(256) k_bwd_act_rows(const GemmArgs p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long rows = p.offsets[p.E];
  const int I = p.I;
  const bool gated = act_gated(p.act);
  const int ld = gated ? 2 * I : I;                 // dGU: [dg | du] rows, or du rows (ungated)
  const int dcol = gated ? I : 0;                   // du's first column in a dGU row
  for (long r = (long)blockIdx.x * 4 + wave; r < rows; r += (long)gridDim.x * 4) {
    const float w = p.topk_w[p.row_slot[r]];
    const float* Pr = p.P + (size_t)r * I;
    const float* Gr = p.GU + (size_t)r * (2 * I);
    const float* Ur = Gr + I;
    float dot = 0.f;
    for (int c = lane * 4; c < I; c += 256) {
      const float4 p4 = *reinterpret_cast<const float4*>(Pr + c);
      const float4 u4 = *reinterpret_cast<const float4*>(Ur + c);
      const float4 g4 = gated ? *reinterpret_cast<const float4*>(Gr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      const float Pv[4] = {p4.x, p4.y, p4.z, p4.w}, Uv[4] = {u4.x, u4.y, u4.z, u4.w};
      const float Gv[4] = {g4.x, g4.y, g4.z, g4.w};
      float hw[4], dg[4], du[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float hf, fg, fu;
        if (gated) {
          gated_act_grad(Gv[j], Uv[j], p.act, p.act_limit, hf, fg, fu);
        } else {
          hf = relu2(Uv[j]);
          fg = 0.f;
          fu = relu2_grad(Uv[j]);
        }
        const float hv = bf16_to_f32(f32_to_bf16(hf));
        dot += hv * Pv[j];
        hw[j] = w * hv;
        dg[j] = w * Pv[j] * fg;
        du[j] = w * Pv[j] * fu;
      }
      uint2 hi, lo;
      split4(hw, hi, lo);
      *reinterpret_cast<uint2*>(p.hw + (size_t)r * I + c) = hi;
      *reinterpret_cast<uint2*>(p.hw_lo + (size_t)r * I + c) = lo;
      if (gated) {
        split4(dg, hi, lo);
        *reinterpret_cast<uint2*>(p.dGU + (size_t)r * ld + c) = hi;
        *reinterpret_cast<uint2*>(p.dGU_lo + (size_t)r * ld + c) = lo;
      }
      split4(du, hi, lo);
      *reinterpret_cast<uint2*>(p.dGU + (size_t)r * ld + dcol + c) = hi;
      *reinterpret_cast<uint2*>(p.dGU_lo + (size_t)r * ld + dcol + c) = lo;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
    if (lane == 0) p.dwt_part[r] = dot;
  }
}

hipError_t launch_bwd_act_rows(const GemmArgs& a, hipStream_t s) {
  const long A = (long)a.T * a.k;
  long blocks = (A + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_bwd_act_rows, dim3((int)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_token_reduce(const GemmArgs& a, const int32_t* slot_row, uint16_t* dX,
                                   float* dtw, hipStream_t s) {
  const long units = (long)a.T * ((a.H / 8 + 63) / 64);
  long blocks = (units + 3) / 4;
  if (blocks > 16384) blocks = 16384;                // one unit per wave up to 8192 tokens of H = 4096
  hipLaunchKernelGGL(k_bwd_token_reduce, dim3((int)blocks), dim3(256), 0, s, a, slot_row, dX, dtw);
  return hipGetLastError();
}

}  // namespace moe
