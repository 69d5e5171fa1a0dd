// Small-token expert MLP (every expert has at most T <= 64 rows): the layer
// is bound by reading each used expert's weights once from HBM, so both
// kernels stream weight rows straight from global memory into MFMA operands
// (no LDS staging) with the few token rows on the narrow side of a
// v_mfma_f32_16x16x32_bf16 ("swap-AB": weights are the 16-row A operand,
// tokens the 16-column B operand, up to four token groups of 16).
//
// Work units are (used expert, slab of output features); a persistent grid
// walks them after building the list of experts that have rows, so experts
// without rows cost nothing.
//
// Each lane reads 32 contiguous bytes of a weight row per step, so one load
// instruction covers 16 rows x 128 bytes (whole cache lines); the two MFMAs of
// a 64-wide k step take the two halves.  Any assignment of contraction indices
// to MFMA k slots gives the same sum as long as both operands use it.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace moe {

#ifndef MOE_DEC_KSPLIT
#define MOE_DEC_KSPLIT 4
#endif
#ifndef MOE_DEC_PF
#define MOE_DEC_PF 4
#endif
constexpr int DEC_NT = 256;            // 4 waves (work-list build, down)
constexpr int DEC_GU_WAVES = MOE_DEC_KSPLIT;   // gate/up: waves splitting the contraction axis
constexpr int DEC_GU_NT = 64 * DEC_GU_WAVES;

// Work list of (expert, group of 16 rows) entries for the experts that have
// rows, in expert order: list[i] = e | (group << 16), i < count.  Returns count
// (at most 4 * E entries: T <= 64).
__device__ int build_group_list(const int32_t* offsets, int E, int* list, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int cnt[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = threadIdx.x * 4 + i;
    cnt[i] = (e < E) ? (offsets[e + 1] - offsets[e] + 15) >> 4 : 0;
    sum += cnt[i];
  }
  int x = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < DEC_NT / 64; ++w) {
    if (w < wave) base += red[w];
    total += red[w];
  }
  int pos = base + x - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    for (int g = 0; g < cnt[i]; ++g) list[pos++] = (threadIdx.x * 4 + i) | (g << 16);
  __syncthreads();
  return total;
}

// The work list, built once per call: wl[0] = entry count, wl[1 + i] = entry i.
__global__ void __launch_bounds__(DEC_NT) k_decode_prep(const int32_t* offsets, int E, int32_t* wl) {
  __shared__ int list[4 * 1024];
  __shared__ int red[8];
  const int n = build_group_list(offsets, E, list, red);
  for (int i = threadIdx.x; i < n; i += DEC_NT) wl[1 + i] = list[i];
  if (threadIdx.x == 0) wl[0] = n;
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// One wave per unit (expert, 16 output features) with the whole contraction
// axis: no LDS, no barriers.  Weight loads for PF k-steps (and the first token
// group's operand) are in flight while the previous steps run on the MFMA.
template <int PF>
struct WaveStream {
  // rows: 16 weight rows per matrix (lane & 15), each lane owns 32 bytes of a 64-wide k step
  // (plain cached loads: measured faster than nontemporal ones for this stream)
  static __device__ __forceinline__ void load(const uint16_t* w, int ks, uint4 (&dst)[2]) {
    const uint4* q = reinterpret_cast<const uint4*>(w + ks * 64);
    dst[0] = q[0];
    dst[1] = q[1];
  }
  static __device__ __forceinline__ void load_x(const uint16_t* x, int ks, uint4 (&dst)[2]) {
    const uint4* q = reinterpret_cast<const uint4*>(x + ks * 64);
    dst[0] = q[0];
    dst[1] = q[1];
  }
};

__device__ __forceinline__ f32x4 mfma2(const uint4 (&a)[2], const uint4 (&b)[2], f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[0]), as_bf16x8(b[0]), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[1]), as_bf16x8(b[1]), c, 0, 0, 0);
}

constexpr int DEC_PF = MOE_DEC_PF;

// Runs step(s) for k-steps 0..n-1 (step kk uses buffer kk % DEC_PF) with the
// loads of step kk + DEC_PF issued right after step kk.  When n is a multiple
// of DEC_PF the steady state has no conditional load, so the in-order vmcnt
// waits the compiler places before each step leave the later buffers in flight
// (a conditional issue makes it wait for every outstanding load instead).
template <class Load, class Step>
__device__ __forceinline__ void stream_steps(int n, Load load, Step step) {
  if (n >= DEC_PF && n % DEC_PF == 0) {
#pragma unroll
    for (int s = 0; s < DEC_PF; ++s) load(s, s);
    for (int ks = 0; ks < n - DEC_PF; ks += DEC_PF) {
#pragma unroll
      for (int s = 0; s < DEC_PF; ++s) {
        step(s);
        load(ks + s + DEC_PF, s);
      }
    }
#pragma unroll
    for (int s = 0; s < DEC_PF; ++s) step(s);
  } else {
#pragma unroll
    for (int s = 0; s < DEC_PF; ++s)
      if (s < n) load(s, s);
    for (int ks = 0; ks < n; ks += DEC_PF) {
#pragma unroll
      for (int s = 0; s < DEC_PF; ++s) {
        if (ks + s < n) {
          step(s);
          if (ks + s + DEC_PF < n) load(ks + s + DEC_PF, s);
        }
      }
    }
  }
}

// Every unit covers one group of up to 16 rows of one expert (lane & 15 is
// the row); lanes past the expert's last row read a valid row (the last one)
// and their output columns are not stored, so no load is predicated and the
// weight prefetch is never drained by a divergent branch.

// gate/up + gated activation: one workgroup per unit (expert, row group, 16 intermediate
// columns); its 4 waves split the contraction axis in 4 and their partial sums
// are added through LDS in wave order before the epilogue.
template <int ACTK>
__device__ __forceinline__ void decode_gateup(const GemmArgs& p) {
  __shared__ f32x4 part[DEC_GU_WAVES - 1][2][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slabs = p.I / 16;
  const int u = blockIdx.x;
  if (u >= p.wlist[0] * slabs) return;                 // whole workgroup: no unit
  const int ent = p.wlist[1 + u / slabs];
  const int e = ent & 0xffff, g = ent >> 16;
  const int i0 = (u % slabs) * 16;
  const int r0 = p.offsets[e] + g * 16, n = min(p.offsets[e + 1] - r0, 16);
  const int ksteps = p.H / 64;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int k_lo = wave_u * ksteps / DEC_GU_WAVES, nks = (wave_u + 1) * ksteps / DEC_GU_WAVES - k_lo;
  const size_t wrow = ((size_t)e * p.I + i0 + (lane & 15)) * p.H + (lane >> 4) * 16 + (size_t)k_lo * 64;
  constexpr bool GATED = act_gated(ACTK);            // ReLU^2 streams W_up only
  const uint16_t* wg = GATED ? p.Wg_t + wrow : nullptr;
  const uint16_t* wu = p.Wu_t + wrow;
  const int t = min(lane & 15, n - 1);
  const uint16_t* xr = p.X + (size_t)p.row_token[r0 + t] * p.H + (lane >> 4) * 16 + (size_t)k_lo * 64;
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
  uint4 bg[DEC_PF][2], bu[DEC_PF][2], bx[DEC_PF][2];
  auto load = [&](int kk, int s) {
    if constexpr (GATED) WaveStream<DEC_PF>::load(wg, kk, bg[s]);
    WaveStream<DEC_PF>::load(wu, kk, bu[s]);
    WaveStream<DEC_PF>::load_x(xr, kk, bx[s]);
  };
  auto step = [&](int s) {
    if constexpr (GATED) ag = mfma2(bg[s], bx[s], ag);
    au = mfma2(bu[s], bx[s], au);
  };
  stream_steps(nks, load, step);
  if (wave > 0) {
    if constexpr (GATED) part[wave - 1][0][lane] = ag;
    part[wave - 1][1][lane] = au;
  }
  __syncthreads();
  if (wave != 0) return;
  // D layout: lane holds row (lane & 15), features 4 * (lane >> 4) + v
  if ((lane & 15) < n) {
#pragma unroll
    for (int w = 0; w < DEC_GU_WAVES - 1; ++w) {
      if constexpr (GATED) ag += part[w][0][lane];
      au += part[w][1][lane];
    }
    float h[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      h[v] = GATED ? gated_act(ag[v], au[v], act_code(ACTK, p.act), p.act_limit) : relu2(au[v]);
    store_bf16x4(p.Hrows + (size_t)(r0 + (lane & 15)) * p.I + i0 + 4 * (lane >> 4), h[0], h[1], h[2], h[3]);
  }
}

__global__ void __launch_bounds__(DEC_GU_NT) k_decode_gateup(const GemmArgs p) { decode_gateup<ACT_SWIGLU>(p); }
// any other gated activation (run-time code)
__global__ void __launch_bounds__(DEC_GU_NT) k_decode_gateup_act(const GemmArgs p) { decode_gateup<ACT_ANY>(p); }
// the ungated ReLU^2 expert (W_up only)
__global__ void __launch_bounds__(DEC_GU_NT) k_decode_up(const GemmArgs p) { decode_gateup<ACT_RELU2>(p); }

// down: one workgroup per (expert, row group, 64 hidden columns), one wave per
// 16 columns over the whole intermediate axis.
__global__ void __launch_bounds__(DEC_NT) k_decode_down(const GemmArgs p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int slabs = p.H / 64;
  const int u = blockIdx.x;
  if (u >= p.wlist[0] * slabs) return;
  const int ent = p.wlist[1 + u / slabs];
  const int e = ent & 0xffff, g = ent >> 16;
  const int h0 = (u % slabs) * 64 + wave * 16;
  const int r0 = p.offsets[e] + g * 16, n = min(p.offsets[e + 1] - r0, 16);
  const int ksteps = p.I / 64;
  const uint16_t* wd = p.Wd_t + ((size_t)e * p.H + h0 + (lane & 15)) * p.I + (lane >> 4) * 16;
  const uint16_t* hr = p.Hrows + (size_t)(r0 + min(lane & 15, n - 1)) * p.I + (lane >> 4) * 16;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint4 bw[DEC_PF][2], bx[DEC_PF][2];
  auto load = [&](int kk, int s) {
    WaveStream<DEC_PF>::load(wd, kk, bw[s]);
    WaveStream<DEC_PF>::load_x(hr, kk, bx[s]);
  };
  auto step = [&](int s) { acc = mfma2(bw[s], bx[s], acc); };
  stream_steps(ksteps, load, step);
  if ((lane & 15) < n)
    store_bf16x4(p.Orows + (size_t)(r0 + (lane & 15)) * p.H + h0 + 4 * (lane >> 4), acc[0], acc[1], acc[2], acc[3]);
}

size_t decode_ws_bytes(int E) { return (size_t)(1 + 4 * E) * sizeof(int32_t); }

hipError_t launch_decode_mlp(const GemmArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_decode_prep, dim3(1), dim3(DEC_NT), 0, s, a.offsets, a.E, a.wlist);
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  // one workgroup per possible unit: at most min(T*k, E) experts with rows, and
  // at most T*k / 16 + (experts with rows) row groups; workgroups past the real
  // unit count exit at once
  const long rows = (long)a.T * a.k;
  const long experts = rows < a.E ? rows : a.E;
  const long groups = rows / 16 + experts;
  hipLaunchKernelGGL(a.act == ACT_SWIGLU ? k_decode_gateup : a.act == ACT_RELU2 ? k_decode_up : k_decode_gateup_act,
                     dim3((unsigned)(groups * (a.I / 16))), dim3(DEC_GU_NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_down, dim3((unsigned)(groups * (a.H / 64))), dim3(DEC_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
