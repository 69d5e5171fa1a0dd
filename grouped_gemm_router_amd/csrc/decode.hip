// Small-token expert MLP (every expert has at most T <= 64 rows): the layer
// is bound by reading each used expert's weights once from HBM.  Both kernels
// stream the weight rows and the few token rows through a small LDS ring per
// wave into v_mfma_f32_16x16x32_bf16 ("swap-AB": 16 weight rows are the A operand,
// up to 16 token rows the B operand), with no barrier inside the stream.
//
// Work units are (used expert, group of up to 16 rows, slab of output features),
// one workgroup each.  A one-workgroup kernel first lists the (expert, row group)
// entries of the experts that have rows, so experts without rows cost nothing;
// the launch covers the most units a call can have, and the workgroups past the
// real count exit at once.
//
// A k step is 64 contraction elements: 128 bytes, one cache line, of each of 16
// rows.  Its rows reach LDS through direct global->LDS loads of whole lines (8
// rows per load instruction), the weights marked non-temporal: measured on this
// part, a row-strided stream read that way runs at about 7.0 TB/s, against 6.2 TB/s
// for 16-byte register loads that cover half of every line per instruction.
// Each wave waits only for its own loads and reads its MFMA operands back with
// 16-byte LDS reads.  Any assignment of contraction indices to MFMA k slots
// gives the same sum as long as both operands use it.
#include <hip/hip_runtime.h>

#include "common.h"
#include "gemm_rows.h"
#include "kernels.h"

namespace moe {

#ifndef MOE_DEC_PF
#define MOE_DEC_PF 2
#endif
constexpr int DEC_NT = 256;            // 4 waves
constexpr int DEC_WAVES = DEC_NT / 64;
constexpr int DEC_PF = MOE_DEC_PF;     // k steps in flight per wave: stages of its ring

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

// One direct global->LDS load, 64 lanes x 16 bytes from base + voff (per lane) to LDS
// [lds, lds + 1024) (lane l at lds + 16 l); NT marks it non-temporal (read once per call).
template <bool NT>
__device__ __forceinline__ void dec_dma16(const uint8_t* base, uint32_t voff, uint32_t lds) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(uniform_ptr(base)),
                 "s"(lds) : "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(uniform_ptr(base)), "s"(lds)
                 : "m0");
}

// One operand of a k step in a ring stage: 16 rows x 128 bytes in 128 16-byte slots.  Load
// instruction i (0, 1) brings rows 8i .. 8i + 7: lane l fetches chunk (l % 8) ^ (l / 8) of row
// 8i + l / 8 into slot 64i + l, so chunk c of row R sits at slot 64 (R / 8) + 8 (R % 8) +
// (c ^ (R % 8)), and the 16-byte reads of an MFMA operand (lane L: row L % 16, chunk 4m + L / 16
// for sub-step m) fall in distinct banks for the eight rows that share a bank group.
struct DecOperand {
  __device__ static int load_row(int lane, int i) { return 8 * i + (lane >> 3); }
  __device__ static uint32_t chunk_byte(int lane) { return (uint32_t)(((lane & 7) ^ (lane >> 3)) * 16); }
  __device__ static int read_slot(int lane, int m) {
    const int R = lane & 15, c = 4 * m + (lane >> 4);
    return 64 * (R >> 3) + 8 * (R & 7) + (c ^ (R & 7));
  }
};

// Waits until this wave's k step is in LDS while `after` (< DEC_PF) later k steps of NPS load
// instructions each may stay in flight (the loads complete in order).
template <int NPS>
__device__ __forceinline__ void dec_wait_steps(int after) {
  static_assert(DEC_PF >= 1 && DEC_PF <= 4 && 3 * NPS < 64, "ring depth");
  if constexpr (DEC_PF >= 4) {
    if (after >= 3) { wait_vmcnt<3 * NPS>(); return; }
  }
  if constexpr (DEC_PF >= 3) {
    if (after >= 2) { wait_vmcnt<2 * NPS>(); return; }
  }
  if constexpr (DEC_PF >= 2) {
    if (after >= 1) { wait_vmcnt<NPS>(); return; }
  }
  wait_vmcnt<0>();
}

// The stream of one wave: nks k steps of NOP operands (16 rows each) through its ring
// (ring[stage][operand][slot]); issue(s, stage) issues the 2 NOP load instructions of step s,
// step(stage) consumes a stage.
template <int NOP, class Issue, class Step>
__device__ __forceinline__ void dec_stream(int nks, uint4 (*ring)[NOP][128], Issue issue, Step step) {
  constexpr int NPS = 2 * NOP;
#pragma unroll
  for (int s = 0; s < DEC_PF; ++s)
    if (s < nks) issue(s, s);
  for (int s = 0; s < nks; ++s) {
    const int st = s % DEC_PF;
    dec_wait_steps<NPS>(min(nks - 1 - s, DEC_PF - 1));
    step(ring[st]);
    if (s + DEC_PF < nks) {
      // every read of this stage is back before its next loads may land
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(s + DEC_PF, st);
    }
  }
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Every unit covers one group of up to 16 rows of one expert (lane & 15 is
// the row); rows past the expert's last row are loaded from the last one and
// their output columns are not stored.

// gate/up + gated activation: one workgroup per unit (expert, row group, 16 intermediate
// columns); its 4 waves split the contraction axis in 4 and their partial sums
// are added through LDS in wave order before the epilogue.
template <int ACTK>
__device__ __forceinline__ void decode_gateup(const GemmArgs& p) {
  constexpr bool GATED = act_gated(ACTK);            // ReLU^2 streams W_up only
  constexpr int NOP = GATED ? 3 : 2;                 // operands: [W_gate,] W_up, token rows
  __shared__ uint4 ring[DEC_WAVES][DEC_PF][NOP][128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slabs = p.I / 16;
  const int u = blockIdx.x;
  if (u >= p.wlist[0] * slabs) return;                 // whole workgroup: no unit
  const int ent = p.wlist[1 + u / slabs];
  const int e = ent & 0xffff, g = ent >> 16;
  const int i0 = (u % slabs) * 16;
  const int r0 = p.offsets[e] + g * 16, n = min(p.offsets[e + 1] - r0, 16);
  const int ksteps = p.H / 64;
  const int k_lo = wave * ksteps / DEC_WAVES, nks = (wave + 1) * ksteps / DEC_WAVES - k_lo;
  // wave-uniform bases (weight rows i0.. of expert e, token matrix X) at this wave's first k
  const size_t wrow0 = ((size_t)e * p.I + i0) * p.H + (size_t)k_lo * 64;
  const uint8_t* wg = reinterpret_cast<const uint8_t*>((GATED ? p.Wg_t : p.Wu_t) + wrow0);
  const uint8_t* wu = reinterpret_cast<const uint8_t*>(p.Wu_t + wrow0);
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(p.X + (size_t)k_lo * 64);
  const uint32_t cb = DecOperand::chunk_byte(lane);
  uint32_t woff[2], xoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = DecOperand::load_row(lane, i);
    woff[i] = (uint32_t)r * (uint32_t)p.H * 2u + cb;
    xoff[i] = (uint32_t)p.row_token[r0 + min(r, n - 1)] * (uint32_t)p.H * 2u + cb;
  }
  uint4(*my)[NOP][128] = ring[wave];
  auto issue = [&](int s, int st) {
    const uint32_t kb = (uint32_t)s * 128u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (GATED) dec_dma16<true>(wg, woff[i] + kb, lds_addr(&my[st][0][64 * i]));
      dec_dma16<true>(wu, woff[i] + kb, lds_addr(&my[st][NOP - 2][64 * i]));
      dec_dma16<false>(xb, xoff[i] + kb, lds_addr(&my[st][NOP - 1][64 * i]));   // reused by every slab
    }
  };
  f32x4 ag = {0.f, 0.f, 0.f, 0.f}, au = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](uint4 (*st)[128]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = DecOperand::read_slot(lane, m);
      const uint4 x = st[NOP - 1][q];
      if constexpr (GATED) ag = mfma16(st[0][q], x, ag);
      au = mfma16(st[NOP - 2][q], x, au);
    }
  };
  dec_stream<NOP>(nks, my, issue, step);
  // partial sums of waves 1-3 in their own rings (their loads have all landed)
  if (wave > 0) {
    my[0][0][lane] = __builtin_bit_cast(uint4, ag);
    my[0][1][lane] = __builtin_bit_cast(uint4, au);
  }
  __syncthreads();
  if (wave != 0) return;
  // D layout: lane holds row (lane & 15), features 4 * (lane >> 4) + v
  if ((lane & 15) < n) {
#pragma unroll
    for (int w = 1; w < DEC_WAVES; ++w) {
      if constexpr (GATED) ag += __builtin_bit_cast(f32x4, ring[w][0][0][lane]);
      au += __builtin_bit_cast(f32x4, ring[w][0][1][lane]);
    }
    float h[4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      h[v] = GATED ? gated_act(ag[v], au[v], act_code(ACTK, p.act), p.act_limit) : relu2(au[v]);
    store_bf16x4(p.Hrows + (size_t)(r0 + (lane & 15)) * p.I + i0 + 4 * (lane >> 4), h[0], h[1], h[2], h[3]);
  }
}

__global__ void __launch_bounds__(DEC_NT) k_decode_gateup(const GemmArgs p) { decode_gateup<ACT_SWIGLU>(p); }
// any other gated activation (run-time code)
__global__ void __launch_bounds__(DEC_NT) k_decode_gateup_act(const GemmArgs p) { decode_gateup<ACT_ANY>(p); }
// the ungated ReLU^2 expert (W_up only)
__global__ void __launch_bounds__(DEC_NT) k_decode_up(const GemmArgs p) { decode_gateup<ACT_RELU2>(p); }

// down: one workgroup per (expert, row group, 64 hidden columns), one wave per
// 16 columns over the whole intermediate axis.
__global__ void __launch_bounds__(DEC_NT) k_decode_down(const GemmArgs p) {
  __shared__ uint4 ring[DEC_WAVES][DEC_PF][2][128];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int slabs = p.H / 64;
  const int u = blockIdx.x;
  if (u >= p.wlist[0] * slabs) return;
  const int ent = p.wlist[1 + u / slabs];
  const int e = ent & 0xffff, g = ent >> 16;
  const int h0 = (u % slabs) * 64 + wave * 16;
  const int r0 = p.offsets[e] + g * 16, n = min(p.offsets[e + 1] - r0, 16);
  const int ksteps = p.I / 64;
  const uint8_t* wd = reinterpret_cast<const uint8_t*>(p.Wd_t + ((size_t)e * p.H + h0) * p.I);
  const uint8_t* hb = reinterpret_cast<const uint8_t*>(p.Hrows);
  const uint32_t cb = DecOperand::chunk_byte(lane);
  uint32_t woff[2], hoff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = DecOperand::load_row(lane, i);
    woff[i] = (uint32_t)r * (uint32_t)p.I * 2u + cb;
    hoff[i] = (uint32_t)(r0 + min(r, n - 1)) * (uint32_t)p.I * 2u + cb;
  }
  uint4(*my)[2][128] = ring[wave];
  auto issue = [&](int s, int st) {
    const uint32_t kb = (uint32_t)s * 128u;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      dec_dma16<true>(wd, woff[i] + kb, lds_addr(&my[st][0][64 * i]));
      dec_dma16<false>(hb, hoff[i] + kb, lds_addr(&my[st][1][64 * i]));   // reused by every slab
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto step = [&](uint4 (*st)[128]) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = DecOperand::read_slot(lane, m);
      acc = mfma16(st[0][q], st[1][q], acc);
    }
  };
  dec_stream<2>(ksteps, my, issue, step);
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
                     dim3((unsigned)(groups * (a.I / 16))), dim3(DEC_NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_down, dim3((unsigned)(groups * (a.H / 64))), dim3(DEC_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
