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

constexpr int DEC_NT = 256;            // 4 waves
constexpr int DEC_GROUPS = DECODE_MAX_T / 16;

// Experts with rows, in expert order: list[0..count).  Returns count.
__device__ int build_active_list(const int32_t* offsets, int E, int* list, int* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int flags[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = threadIdx.x * 4 + i;
    flags[i] = (e < E) && (offsets[e + 1] > offsets[e]);
    sum += flags[i];
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
    if (flags[i]) list[pos++] = threadIdx.x * 4 + i;
  __syncthreads();
  return total;
}

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// One wave per unit (expert, 16 output features) with the whole contraction
// axis: no LDS, no barriers.  Weight loads for PF k-steps (and the first token
// group's operand) are in flight while the previous steps run on the MFMA.
template <int PF>
struct WaveStream {
  // rows: 16 weight rows per matrix (lane & 15), each lane owns 32 bytes of a 64-wide k step
  static __device__ __forceinline__ void load(const uint16_t* w, int ks, uint4 (&dst)[2]) {
    const uint4* q = reinterpret_cast<const uint4*>(w + ks * 64);
    dst[0] = ldg_nt(q);
    dst[1] = ldg_nt(q + 1);
  }
  static __device__ __forceinline__ void load_x(const uint16_t* x, int ks, uint4 (&dst)[2]) {
    if (x) {
      const uint4* q = reinterpret_cast<const uint4*>(x + ks * 64);
      dst[0] = q[0];
      dst[1] = q[1];
    } else {
      dst[0] = dst[1] = make_uint4(0, 0, 0, 0);
    }
  }
};

__device__ __forceinline__ f32x4 mfma2(const uint4 (&a)[2], const uint4 (&b)[2], f32x4 c) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[0]), as_bf16x8(b[0]), c, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[1]), as_bf16x8(b[1]), c, 0, 0, 0);
}

constexpr int DEC_PF = 4;

// gate/up + SwiGLU: unit = (expert, 16 intermediate columns), one wave.
__global__ void __launch_bounds__(DEC_NT) k_decode_gateup(const GemmArgs p) {
  __shared__ int list[1024];
  __shared__ int red[8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nact = build_active_list(p.offsets, p.E, list, red);
  const int slabs = p.I / 16;
  const int units = nact * slabs;
  const int ksteps = p.H / 64;
  for (int u = blockIdx.x * 4 + wave; u < units; u += gridDim.x * 4) {
    const int e = list[u / slabs];
    const int i0 = (u % slabs) * 16;
    const int r0 = p.offsets[e], n = p.offsets[e + 1] - r0;
    const int ngroups = (n + 15) >> 4;
    const size_t wrow = ((size_t)e * p.I + i0 + (lane & 15)) * p.H + (lane >> 4) * 16;
    const uint16_t* wg = p.Wg_t + wrow;
    const uint16_t* wu = p.Wu_t + wrow;
    const uint16_t* xr[DEC_GROUPS];
#pragma unroll
    for (int g = 0; g < DEC_GROUPS; ++g) {
      int t = g * 16 + (lane & 15);
      xr[g] = (t < n) ? p.X + (size_t)p.row_token[r0 + t] * p.H + (lane >> 4) * 16 : nullptr;
    }
    f32x4 ag[DEC_GROUPS], au[DEC_GROUPS];
#pragma unroll
    for (int g = 0; g < DEC_GROUPS; ++g) ag[g] = au[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 bg[DEC_PF][2], bu[DEC_PF][2], bx[DEC_PF][2];
#pragma unroll
    for (int s = 0; s < DEC_PF; ++s) {
      if (s < ksteps) {
        WaveStream<DEC_PF>::load(wg, s, bg[s]);
        WaveStream<DEC_PF>::load(wu, s, bu[s]);
        WaveStream<DEC_PF>::load_x(xr[0], s, bx[s]);
      }
    }
    for (int ks = 0; ks < ksteps; ks += DEC_PF) {
#pragma unroll
      for (int s = 0; s < DEC_PF; ++s) {
        const int kk = ks + s;
        if (kk < ksteps) {
          ag[0] = mfma2(bg[s], bx[s], ag[0]);
          au[0] = mfma2(bu[s], bx[s], au[0]);
#pragma unroll
          for (int g = 1; g < DEC_GROUPS; ++g) {
            if (g < ngroups) {
              uint4 x[2];
              WaveStream<DEC_PF>::load_x(xr[g], kk, x);
              ag[g] = mfma2(bg[s], x, ag[g]);
              au[g] = mfma2(bu[s], x, au[g]);
            }
          }
          const int nk = kk + DEC_PF;
          if (nk < ksteps) {
            WaveStream<DEC_PF>::load(wg, nk, bg[s]);
            WaveStream<DEC_PF>::load(wu, nk, bu[s]);
            WaveStream<DEC_PF>::load_x(xr[0], nk, bx[s]);
          }
        }
      }
    }
    // D layout: lane holds token (lane & 15), features 4 * (lane >> 4) + v
#pragma unroll
    for (int g = 0; g < DEC_GROUPS; ++g) {
      const int row = g * 16 + (lane & 15);
      if (g < ngroups && row < n) {
        float h[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) h[v] = silu_f32(ag[g][v]) * au[g][v];
        store_bf16x4(p.Hrows + (size_t)(r0 + row) * p.I + i0 + 4 * (lane >> 4), h[0], h[1], h[2], h[3]);
      }
    }
  }
}

// down: unit = (expert, 16 hidden columns), one wave, whole intermediate axis.
__global__ void __launch_bounds__(DEC_NT) k_decode_down(const GemmArgs p) {
  __shared__ int list[1024];
  __shared__ int red[8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nact = build_active_list(p.offsets, p.E, list, red);
  const int slabs = p.H / 16;
  const int units = nact * slabs;
  const int ksteps = p.I / 64;
  for (int u = blockIdx.x * 4 + wave; u < units; u += gridDim.x * 4) {
    const int e = list[u / slabs];
    const int h0 = (u % slabs) * 16;
    const int r0 = p.offsets[e], n = p.offsets[e + 1] - r0;
    const int ngroups = (n + 15) >> 4;
    const uint16_t* wd = p.Wd_t + ((size_t)e * p.H + h0 + (lane & 15)) * p.I + (lane >> 4) * 16;
    const uint16_t* hr[DEC_GROUPS];
#pragma unroll
    for (int g = 0; g < DEC_GROUPS; ++g) {
      int t = g * 16 + (lane & 15);
      hr[g] = (t < n) ? p.Hrows + (size_t)(r0 + t) * p.I + (lane >> 4) * 16 : nullptr;
    }
    f32x4 acc[DEC_GROUPS];
#pragma unroll
    for (int g = 0; g < DEC_GROUPS; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint4 bw[DEC_PF][2], bx[DEC_PF][2];
#pragma unroll
    for (int s = 0; s < DEC_PF; ++s) {
      if (s < ksteps) {
        WaveStream<DEC_PF>::load(wd, s, bw[s]);
        WaveStream<DEC_PF>::load_x(hr[0], s, bx[s]);
      }
    }
    for (int ks = 0; ks < ksteps; ks += DEC_PF) {
#pragma unroll
      for (int s = 0; s < DEC_PF; ++s) {
        const int kk = ks + s;
        if (kk < ksteps) {
          acc[0] = mfma2(bw[s], bx[s], acc[0]);
#pragma unroll
          for (int g = 1; g < DEC_GROUPS; ++g) {
            if (g < ngroups) {
              uint4 x[2];
              WaveStream<DEC_PF>::load_x(hr[g], kk, x);
              acc[g] = mfma2(bw[s], x, acc[g]);
            }
          }
          const int nk = kk + DEC_PF;
          if (nk < ksteps) {
            WaveStream<DEC_PF>::load(wd, nk, bw[s]);
            WaveStream<DEC_PF>::load_x(hr[0], nk, bx[s]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < DEC_GROUPS; ++g) {
      const int row = g * 16 + (lane & 15);
      if (g < ngroups && row < n)
        store_bf16x4(p.Orows + (size_t)(r0 + row) * p.H + h0 + 4 * (lane >> 4), acc[g][0], acc[g][1], acc[g][2],
                     acc[g][3]);
    }
  }
}

// Blocks of 4 waves; up to 8 blocks per CU resident, one pass over the units.
static int decode_grid(long wave_units_upper) {
  long blocks = (wave_units_upper + 3) / 4;
  long cap = (long)num_cus() * 8;
  long g = blocks < cap ? blocks : cap;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_decode_mlp(const GemmArgs& a, hipStream_t s) {
  long active_upper = (long)a.T * a.k < a.E ? (long)a.T * a.k : a.E;
  hipLaunchKernelGGL(k_decode_gateup, dim3(decode_grid(active_upper * (a.I / 16))), dim3(DEC_NT), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_decode_down, dim3(decode_grid(active_upper * (a.H / 16))), dim3(DEC_NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
