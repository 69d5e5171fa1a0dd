// bf16 grouped GEMMs of the MoE layer: forward gate/up + SwiGLU, forward down,
// and the five GEMMs of the backward.  See grouped_gemm.h for the template.
#include "grouped_gemm.h"
#include "kernels.h"

namespace moe {

using CfgMain = TileCfg<256, 256, 2, 2>;

// ------------------------------------------------------------------------
// Operand sources
// ------------------------------------------------------------------------
// Token rows X[row_token[r]] (contraction axis H) for the rows of a tile.
struct SrcXRows {
  __device__ static int ksplit(const GemmArgs& p) { return p.H; }
  __device__ static long delta(const GemmArgs&) { return 0; }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int row) {
    int r = t.m0 + row;
    return r < t.m_end ? p.X + (size_t)p.row_token[r] * p.H : nullptr;
  }
};
struct SrcDYRows {
  __device__ static int ksplit(const GemmArgs& p) { return p.H; }
  __device__ static long delta(const GemmArgs&) { return 0; }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int row) {
    int r = t.m0 + row;
    return r < t.m_end ? p.dY + (size_t)p.row_token[r] * p.H : nullptr;
  }
};
// Expert-major activation rows h (contraction axis I).
struct SrcHRows {
  __device__ static int ksplit(const GemmArgs& p) { return p.I; }
  __device__ static long delta(const GemmArgs&) { return 0; }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int row) {
    int r = t.m0 + row;
    return r < t.m_end ? p.Hrows + (size_t)r * p.I : nullptr;
  }
};
// Expert-major gradient rows [dg | du] (contraction axis 2I).
struct SrcDGURows {
  __device__ static int ksplit(const GemmArgs& p) { return 2 * p.I; }
  __device__ static long delta(const GemmArgs&) { return 0; }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int row) {
    int r = t.m0 + row;
    return r < t.m_end ? p.dGU + (size_t)r * 2 * p.I : nullptr;
  }
};
// Gate and up weight rows of the packed [E, I, H] layout, interleaved per wave
// column group: the first half of every WTN rows are gate columns, the second
// half the up columns of the same intermediate indices.
template <class C>
struct SrcGateUpW {
  __device__ static int ksplit(const GemmArgs& p) { return p.H; }
  __device__ static long delta(const GemmArgs&) { return 0; }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int rr) {
    constexpr int half = C::WTN / 2;
    int g = rr / C::WTN, within = rr % C::WTN;
    bool up = within >= half;
    int col = t.nt * (C::BN / 2) + g * half + (within % half);
    return col < p.I ? (up ? p.Wu_t : p.Wg_t) + ((size_t)t.e * p.I + col) * p.H : nullptr;
  }
};
// Packed down weights [E, H, I]: output column n = hidden index.
struct SrcDownW {
  __device__ static int ksplit(const GemmArgs& p) { return p.I; }
  __device__ static long delta(const GemmArgs&) { return 0; }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int rr) {
    int n = t.n0 + rr;
    return n < p.H ? p.Wd_t + ((size_t)t.e * p.H + n) * p.I : nullptr;
  }
};
// W_down in the math layout [E, I, H] read as [E, N = I, K = H] (P = dY W_down^T).
struct SrcDownWT {
  __device__ static int ksplit(const GemmArgs& p) { return p.H; }
  __device__ static long delta(const GemmArgs&) { return 0; }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int rr) {
    int n = t.n0 + rr;
    return n < p.I ? p.Wd + ((size_t)t.e * p.I + n) * p.H : nullptr;
  }
};
// [W_gate | W_up] in the math layout [E, H, I] read as [E, N = H, K = 2I]:
// columns k >= I come from W_up at the same offset.
struct SrcGateUpWT {
  __device__ static int ksplit(const GemmArgs& p) { return p.I; }
  __device__ static long delta(const GemmArgs& p) { return (long)(p.Wu - p.Wg); }
  __device__ static const uint16_t* rows(const GemmArgs& p, const Tile& t, int rr) {
    int n = t.n0 + rr;
    return n < p.H ? p.Wg + ((size_t)t.e * p.H + n) * p.I : nullptr;
  }
};
// Row sources of the weight-gradient GEMMs (rows are the contraction index).
struct MNSrcH {
  static constexpr bool SCALED = false;
  __device__ static const uint16_t* row(const GemmArgs& p, const Tile&, int r, int) {
    return p.Hrows + (size_t)r * p.I;
  }
  __device__ static float scale(const GemmArgs&, int) { return 1.f; }
};
struct MNSrcDO {  // dO = bf16(w * dY[token])
  static constexpr bool SCALED = true;
  __device__ static const uint16_t* row(const GemmArgs& p, const Tile&, int r, int) {
    return p.dY + (size_t)p.row_token[r] * p.H;
  }
  __device__ static float scale(const GemmArgs& p, int r) { return p.topk_w[p.row_slot[r]]; }
};
struct MNSrcX {
  static constexpr bool SCALED = false;
  __device__ static const uint16_t* row(const GemmArgs& p, const Tile&, int r, int) {
    return p.X + (size_t)p.row_token[r] * p.H;
  }
  __device__ static float scale(const GemmArgs&, int) { return 1.f; }
};
// [dg | du] rows: the bf16 values in the first pass, their bf16 remainders in the second.
struct MNSrcDGU {
  static constexpr bool SCALED = false;
  __device__ static const uint16_t* row(const GemmArgs& p, const Tile&, int r, int phase) {
    return (phase ? p.dGU_lo : p.dGU) + (size_t)r * 2 * p.I;
  }
  __device__ static float scale(const GemmArgs&, int) { return 1.f; }
};

// ------------------------------------------------------------------------
// Ops: schedule + loaders + epilogue of each GEMM
// ------------------------------------------------------------------------
template <class C, class SrcA, class SrcB>
struct RowOpsBase {
  static constexpr int PHASES = 1;
  using Sched = RowGroups<C::BM, C::BN, C::NT>;
  using ALoad = KRows<C::BM, C::NT, SrcA, GemmArgs>;
  using BLoad = KRows<C::BN, C::NT, SrcB, GemmArgs>;
  __device__ static void init_loaders(ALoad& al, BLoad& bl, const GemmArgs& p, const Tile& t) {
    al.init(p, t);
    bl.init(p, t);
  }
};

// h = bf16(silu(X Wg) * (X Wu))
template <class C>
struct FwdGateUpOps : RowOpsBase<C, SrcXRows, SrcGateUpW<C>> {
  __device__ static void init_sched(typename RowOpsBase<C, SrcXRows, SrcGateUpW<C>>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, 2 * p.I, p.H, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane) {
    const int hcol0 = t.nt * (C::BN / 2) + wn * (C::WTN / 2) + (lane >> 5) * 4;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int r = t.m0 + Frag<C>::row(wm, fm, lane);
      if (r >= t.m_end) continue;
      uint16_t* out = p.Hrows + (size_t)r * p.I + hcol0;
#pragma unroll
      for (int fn = 0; fn < C::FN / 2; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (hcol0 + fn * 32 + q * 8 >= p.I) continue;
          float h[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            h[j] = silu_f32(acc[fm][fn][4 * q + j]) * acc[fm][fn + C::FN / 2][4 * q + j];
          store_bf16x4(out + fn * 32 + q * 8, h[0], h[1], h[2], h[3]);
        }
    }
  }
};

// Plain store of the tile (bf16 or fp32) to out[r * ld + n], rows of the expert only.
template <class C, typename T>
__device__ __forceinline__ void store_rows(T* base, int ld, int ncols, const Tile& t,
                                           f32x16 (&acc)[C::FM][C::FN], int wm, int wn, int lane) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int r = t.m0 + Frag<C>::row(wm, fm, lane);
    if (r >= t.m_end) continue;
    T* out = base + (size_t)r * ld;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = t.n0 + Frag<C>::col(wn, fn, q, lane);
        if (n >= ncols) continue;
        if constexpr (sizeof(T) == 2) {
          store_bf16x4(reinterpret_cast<uint16_t*>(out + n), acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1],
                       acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]);
        } else {
          *reinterpret_cast<float4*>(out + n) =
              make_float4(acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]);
        }
      }
  }
}

// O = bf16(h Wd)
template <class C>
struct FwdDownOps : RowOpsBase<C, SrcHRows, SrcDownW> {
  __device__ static void init_sched(typename RowOpsBase<C, SrcHRows, SrcDownW>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, p.H, p.I, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane) {
    store_rows<C, uint16_t>(p.Orows, p.H, p.H, t, acc, wm, wn, lane);
  }
};

// P = dY[token] W_down^T (fp32)
template <class C>
struct BwdPOps : RowOpsBase<C, SrcDYRows, SrcDownWT> {
  __device__ static void init_sched(typename RowOpsBase<C, SrcDYRows, SrcDownWT>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, p.I, p.H, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane) {
    store_rows<C, float>(p.P, p.I, p.I, t, acc, wm, wn, lane);
  }
};

// v = hi + lo with hi = bf16(v), lo = bf16(v - hi): stores both (4 values).
__device__ __forceinline__ void store_split4(uint16_t* hi, uint16_t* lo, const float (&v)[4]) {
  uint2 h, l;
  h.x = pack_bf16x2(v[0], v[1]);
  h.y = pack_bf16x2(v[2], v[3]);
  l.x = pack_bf16x2(v[0] - bf16_to_f32(h.x & 0xffffu), v[1] - bf16_to_f32(h.x >> 16));
  l.y = pack_bf16x2(v[2] - bf16_to_f32(h.y & 0xffffu), v[3] - bf16_to_f32(h.y >> 16));
  *reinterpret_cast<uint2*>(hi) = h;
  *reinterpret_cast<uint2*>(lo) = l;
}

// Recompute G, U; with P give h, the router-weight partial sums <h, P>, dg and du.
template <class C>
struct BwdRecomputeOps : RowOpsBase<C, SrcXRows, SrcGateUpW<C>> {
  __device__ static void init_sched(typename RowOpsBase<C, SrcXRows, SrcGateUpW<C>>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, 2 * p.I, p.H, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane) {
    const int hcol0 = t.nt * (C::BN / 2) + wn * (C::WTN / 2) + (lane >> 5) * 4;
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int r = t.m0 + Frag<C>::row(wm, fm, lane);
      const bool rv = r < t.m_end;
      float dot = 0.f;
      if (rv) {
        const float w = p.topk_w[p.row_slot[r]];
        const float* Prow = p.P + (size_t)r * p.I + hcol0;
        uint16_t* hrow = p.Hrows + (size_t)r * p.I + hcol0;
        uint16_t* grow = p.dGU + (size_t)r * 2 * p.I + hcol0;
        uint16_t* lrow = p.dGU_lo + (size_t)r * 2 * p.I + hcol0;
#pragma unroll
        for (int fn = 0; fn < C::FN / 2; ++fn)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int o = fn * 32 + q * 8;
            if (hcol0 + o >= p.I) continue;
            const float4 P4 = *reinterpret_cast<const float4*>(Prow + o);
            const float Pv[4] = {P4.x, P4.y, P4.z, P4.w};
            float hv[4], dg[4], du[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float g = acc[fm][fn][4 * q + j], u = acc[fm][fn + C::FN / 2][4 * q + j];
              const float sg = sigmoid_f32(g);
              hv[j] = bf16_to_f32(f32_to_bf16(g * sg * u));
              dot += hv[j] * Pv[j];
              const float dh = w * Pv[j];
              du[j] = dh * (g * sg);
              dg[j] = dh * u * (sg * (1.f + g * (1.f - sg)));
            }
            store_bf16x4(hrow + o, hv[0], hv[1], hv[2], hv[3]);
            store_split4(grow + o, lrow + o, dg);
            store_split4(grow + p.I + o, lrow + p.I + o, du);
          }
      }
      // the other half of this row's columns sits in lane ^ 32
      dot += __shfl_xor(dot, 32, 64);
      if (rv && lane < 32) p.dwt_part[(size_t)r * p.nparts + t.nt * C::WAVES_N + wn] = dot;
    }
  }
};

// dXr = [dg | du] [W_gate | W_up]^T (fp32 rows)
template <class C>
struct BwdDXOps : RowOpsBase<C, SrcDGURows, SrcGateUpWT> {
  __device__ static void init_sched(typename RowOpsBase<C, SrcDGURows, SrcGateUpWT>::Sched& s,
                                    const GemmArgs& p, int* pre, int* red) {
    s.init(p.offsets, p.E, p.H, 2 * p.I, pre, red);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane) {
    store_rows<C, float>(p.dXr, p.H, p.H, t, acc, wm, wn, lane);
  }
};

template <class C, class SrcA, class SrcB>
struct WgOpsBase {
  static constexpr int PHASES = 1;
  using Sched = WeightGrad<C::BM, C::BN, C::NT>;
  using ALoad = MNRows<C::BM, C::NT, SrcA, GemmArgs>;
  using BLoad = MNRows<C::BN, C::NT, SrcB, GemmArgs>;
};

// Weight-gradient tile store: out[e][m][n] for m < M (n already split by caller).
template <class C>
__device__ __forceinline__ void store_wg(uint16_t* out0, uint16_t* out1, int nsplit, int M, int N,
                                         const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                                         int lane) {
#pragma unroll
  for (int fm = 0; fm < C::FM; ++fm) {
    const int m = t.m0 + Frag<C>::row(wm, fm, lane);
    if (m >= M) continue;
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = t.n0 + Frag<C>::col(wn, fn, q, lane);
        if (n >= N) continue;
        uint16_t* dst = n < nsplit ? out0 + ((size_t)t.e * M + m) * nsplit + n
                                   : out1 + ((size_t)t.e * M + m) * (N - nsplit) + (n - nsplit);
        store_bf16x4(dst, acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                     acc[fm][fn][4 * q + 3]);
      }
  }
}

// dW_down[e] = sum_r h_r^T dO_r   ([I, H])
template <class C>
struct BwdDWDownOps : WgOpsBase<C, MNSrcH, MNSrcDO> {
  using B = WgOpsBase<C, MNSrcH, MNSrcDO>;
  __device__ static void init_sched(typename B::Sched& s, const GemmArgs& p, int*, int*) {
    s.init(p.offsets, p.E, p.I, p.H);
  }
  __device__ static void init_loaders(typename B::ALoad& al, typename B::BLoad& bl, const GemmArgs& p,
                                      const Tile& t) {
    al.init(p, t, t.m0, p.I);
    bl.init(p, t, t.n0, p.H);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane) {
    store_wg<C>(p.dWd, p.dWd, p.H, p.I, p.H, t, acc, wm, wn, lane);
  }
};

// [dW_gate | dW_up][e] = sum_r X_r^T [dg | du]_r   ([H, 2I] split at I)
template <class C>
struct BwdDWGateUpOps : WgOpsBase<C, MNSrcX, MNSrcDGU> {
  using B = WgOpsBase<C, MNSrcX, MNSrcDGU>;
  // dg and du enter as bf16 value + bf16 remainder: two passes over the rows
  static constexpr int PHASES = 2;
  __device__ static void init_sched(typename B::Sched& s, const GemmArgs& p, int*, int*) {
    s.init(p.offsets, p.E, p.H, 2 * p.I);
  }
  __device__ static void init_loaders(typename B::ALoad& al, typename B::BLoad& bl, const GemmArgs& p,
                                      const Tile& t) {
    al.init(p, t, t.m0, p.H);
    bl.init(p, t, t.n0, 2 * p.I);
  }
  __device__ static void epilogue(const GemmArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN],
                                  int wm, int wn, int lane) {
    store_wg<C>(p.dWg, p.dWu, p.I, p.H, 2 * p.I, t, acc, wm, wn, lane);
  }
};

// ------------------------------------------------------------------------
// Kernels and launchers
// ------------------------------------------------------------------------
#define MOE_GEMM_KERNEL(NAME, OPS)                                                 \
  __global__ void __launch_bounds__(CfgMain::NT) NAME(const GemmArgs p) {          \
    grouped_gemm_body<CfgMain, OPS<CfgMain>, GemmArgs>(p);                         \
  }

MOE_GEMM_KERNEL(k_fwd_gateup, FwdGateUpOps)
MOE_GEMM_KERNEL(k_fwd_down, FwdDownOps)
MOE_GEMM_KERNEL(k_bwd_p, BwdPOps)
MOE_GEMM_KERNEL(k_bwd_recompute, BwdRecomputeOps)
MOE_GEMM_KERNEL(k_bwd_dx_rows, BwdDXOps)
MOE_GEMM_KERNEL(k_bwd_dw_down, BwdDWDownOps)
MOE_GEMM_KERNEL(k_bwd_dw_gateup, BwdDWGateUpOps)

template <class C>
static int row_grid(const GemmArgs& a, int N) {
  long A = (long)a.T * a.k;
  long mt = A / C::BM + (a.E < A ? a.E : A) + 1;
  long tiles = mt * ((N + C::BN - 1) / C::BN);
  long cap = (long)num_cus();            // one 132 KB-LDS block per CU
  long g = tiles < cap ? tiles : cap;
  return (int)((g + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
}
template <class C>
static int wg_grid(const GemmArgs& a, int M, int N) {
  long tiles = (long)a.E * ((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
  long cap = (long)num_cus();
  long g = tiles < cap ? tiles : cap;
  return (int)((g + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
}

hipError_t launch_fwd_gateup(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_fwd_gateup, dim3(row_grid<CfgMain>(a, 2 * a.I)), dim3(CfgMain::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_fwd_down(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_fwd_down, dim3(row_grid<CfgMain>(a, a.H)), dim3(CfgMain::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bwd_p(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_p, dim3(row_grid<CfgMain>(a, a.I)), dim3(CfgMain::NT), 0, s, a);
  return hipGetLastError();
}
int bwd_nparts(int I) {
  return ((2 * I + CfgMain::BN - 1) / CfgMain::BN) * CfgMain::WAVES_N;
}
hipError_t launch_bwd_recompute(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_recompute, dim3(row_grid<CfgMain>(a, 2 * a.I)), dim3(CfgMain::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bwd_dx_rows(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_dx_rows, dim3(row_grid<CfgMain>(a, a.H)), dim3(CfgMain::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bwd_dw_down(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_dw_down, dim3(wg_grid<CfgMain>(a, a.I, a.H)), dim3(CfgMain::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_bwd_dw_gateup(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_bwd_dw_gateup, dim3(wg_grid<CfgMain>(a, a.H, 2 * a.I)), dim3(CfgMain::NT), 0, s, a);
  return hipGetLastError();
}

// dX[t] = bf16(sum_j dXr[slot_row[t*k+j]]), d_topk_w[t,j] = sum of the row's partials.
__global__ void __launch_bounds__(256) k_bwd_token_reduce(const GemmArgs p, const int32_t* slot_row,
                                                          uint16_t* dX, float* dtw) {
  const int chunks = p.H / 8;
  const long total = (long)p.T * chunks;
  for (long i = blockIdx.x * 256L + threadIdx.x; i < total; i += (long)gridDim.x * 256) {
    int t = (int)(i / chunks), c = (int)(i % chunks);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j = 0; j < p.k; ++j) {
      int r = slot_row[t * p.k + j];
      const float4* src = reinterpret_cast<const float4*>(p.dXr + (size_t)r * p.H + c * 8);
      float4 a = src[0], b = src[1];
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(dX + (size_t)t * p.H + c * 8) = o;
    for (int j = c; j < p.k; j += chunks) {
      int r = slot_row[t * p.k + j];
      float s = 0.f;
      for (int q = 0; q < p.nparts; ++q) s += p.dwt_part[(size_t)r * p.nparts + q];
      dtw[t * p.k + j] = s;
    }
  }
}

hipError_t launch_bwd_token_reduce(const GemmArgs& a, const int32_t* slot_row, uint16_t* dX,
                                   float* dtw, hipStream_t s) {
  long total = (long)a.T * (a.H / 8);
  long blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_bwd_token_reduce, dim3((int)blocks), dim3(256), 0, s, a, slot_row, dX, dtw);
  return hipGetLastError();
}

}  // namespace moe
