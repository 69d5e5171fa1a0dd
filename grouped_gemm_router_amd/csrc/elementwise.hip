// Memory-bound kernels of the MoE layer on gfx950: weighted combine, weight
// packing (transpose to contraction-contiguous) and MXFP8 quantisation.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Combine: Y[t] = bf16(sum_j w[t,j] * O[slot_row[t*k+j]]), fp32, j ascending.
// One thread per 8 consecutive outputs (16-byte loads and stores); the rows of
// four slots are loaded together, then added in slot order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void combine_add(float (&acc)[8], float wj, const uint4& v) {
  const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] += wj * bf16_to_f32(d[q] & 0xffffu);
    acc[2 * q + 1] += wj * bf16_to_f32(d[q] >> 16);
  }
}

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
// 16-byte load with the nontemporal hint: the O rows are read once, and streaming them past
// the caches took the C3 combine from 158 to 117 us
__device__ __forceinline__ uint4 load_nt(const uint16_t* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p)));
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&a)[8]) {
  return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
}

// One wave per (token, slice of 128 16-byte chunks): the token's k row indices and weights
// are wave-uniform (scalar loads), and each lane sums two chunks, issuing the loads of four
// rows for both before it adds them.  A slot whose row index is negative (dispatch skipped an
// out-of-range expert id) adds nothing (row 0 is loaded in its place, never added).
constexpr int COMBINE_SLICE = 128;          // chunks of 8 bf16 per wave unit (two per lane)

__global__ void __launch_bounds__(256) k_combine(const uint16_t* __restrict__ O, const int32_t* __restrict__ slot_row,
                                                 const float* __restrict__ w, int T, int k, int H,
                                                 uint16_t* __restrict__ Y) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chunks = H / 8;
  const int slices = (chunks + COMBINE_SLICE - 1) / COMBINE_SLICE;
  const long units = (long)T * slices;
  for (long u = (long)blockIdx.x * 4 + wave; u < units; u += (long)gridDim.x * 4) {
    const int t = (int)(u / slices), sl = (int)(u - (long)t * slices);
    const int32_t* sr = slot_row + (size_t)t * k;
    const float* wt = w + (size_t)t * k;
    const int c0 = sl * COMBINE_SLICE + lane, c1 = c0 + 64;
    const bool has0 = c0 < chunks, has1 = c1 < chunks;
    const int cc0 = has0 ? c0 : 0, cc1 = has1 ? c1 : 0;   // in-bounds reads for idle lanes
    float a0[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}, a1[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int j = 0;
    for (; j + 4 <= k; j += 4) {
      uint4 v0[4], v1[4];
      int rr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        rr[q] = sr[j + q];
        const uint16_t* row = O + (size_t)max(rr[q], 0) * H;
        v0[q] = load_nt(row + cc0 * 8);
        v1[q] = load_nt(row + cc1 * 8);
      }
      __builtin_amdgcn_sched_barrier(0);           // all eight loads in flight before the adds
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (rr[q] < 0) continue;
        combine_add(a0, wt[j + q], v0[q]);
        combine_add(a1, wt[j + q], v1[q]);
      }
    }
    for (; j < k; ++j) {
      const int r = sr[j];
      if (r < 0) continue;
      const uint16_t* row = O + (size_t)r * H;
      combine_add(a0, wt[j], load_nt(row + cc0 * 8));
      combine_add(a1, wt[j], load_nt(row + cc1 * 8));
    }
    uint16_t* yr = Y + (size_t)t * H;
    if (has0) *reinterpret_cast<uint4*>(yr + c0 * 8) = pack_bf16x8(a0);
    if (has1) *reinterpret_cast<uint4*>(yr + c1 * 8) = pack_bf16x8(a1);
  }
}

static int grid_for(long work, int per_block, int cap) {
  long b = (work + per_block - 1) / per_block;
  if (b > cap) b = cap;
  return (int)(b < 1 ? 1 : b);
}

hipError_t launch_combine(const uint16_t* O, const int32_t* slot_row, const float* w, int T, int k, int H,
                          uint16_t* Y, hipStream_t s) {
  const long units = (long)T * ((H / 8 + COMBINE_SLICE - 1) / COMBINE_SLICE);
  hipLaunchKernelGGL(k_combine, dim3(grid_for(units, 4, 8192)), dim3(256), 0, s, O, slot_row, w, T, k, H, Y);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Packing: W [E, K, N] -> Wt [E, N, K] (bf16), 64x64 tiles through LDS.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_pack(const uint16_t* __restrict__ W, int K, int N,
                                              uint16_t* __restrict__ Wt) {
  __shared__ uint16_t tile[64][66];
  const int e = blockIdx.z;
  const int k0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  const uint16_t* src = W + (size_t)e * K * N;
  uint16_t* dst = Wt + (size_t)e * K * N;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    int kk = i / 64, nn = i % 64;
    tile[kk][nn] = src[(size_t)(k0 + kk) * N + n0 + nn];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    int nn = i / 64, kk = i % 64;
    dst[(size_t)(n0 + nn) * K + k0 + kk] = tile[kk][nn];
  }
}

hipError_t launch_pack(const uint16_t* W, int E, int K, int N, uint16_t* Wt, hipStream_t s) {
  hipLaunchKernelGGL(k_pack, dim3(N / 64, K / 64, E), dim3(256), 0, s, W, K, N, Wt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// MXFP8 quantisation (OCP MX v1.0 section 6.3) of 32-element blocks along rows:
// scale exponent = floor(log2(amax)) - 8 clamped to [-127, 127] (byte 0 for an
// all-zero block), elements rounded to E4M3FN to nearest even, saturating.
// One thread per block of 32.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int floor_log2_f32(float a) {  // a > 0, finite
  uint32_t u = __float_as_uint(a);
  int ex = (int)(u >> 23);
  if (ex == 0) return -118 - __builtin_clz(u & 0x7fffffu);  // subnormal: mantissa * 2^-149
  return ex - 127;
}

// Four values already scaled by 2^-s to fp8 codes: clamped to +-448 (the
// saturating rule), then converted by v_cvt_pk_fp8_f32 (OCP E4M3 on gfx950,
// round to nearest even; E4M3 subnormals are multiples of 2^-9).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  auto sat = [](float x) { return __builtin_fminf(__builtin_fmaxf(x, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), w, true);
  return (uint32_t)w;
}

__global__ void __launch_bounds__(256) k_mx_quantize(const uint16_t* __restrict__ x, long nblocks,
                                                     uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  for (long b = blockIdx.x * 256L + threadIdx.x; b < nblocks; b += (long)gridDim.x * 256) {
    const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
    uint32_t d[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint4 v = src[i];
      d[4 * i] = v.x; d[4 * i + 1] = v.y; d[4 * i + 2] = v.z; d[4 * i + 3] = v.w;
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      amax = fmaxf(amax, fmaxf(fabsf(bf16_to_f32(d[i] & 0xffffu)), fabsf(bf16_to_f32(d[i] >> 16))));
    uint32_t out[8];
    uint8_t sbyte = 0;
    if (amax > 0.f) {
      int s = floor_log2_f32(amax) - 8;
      s = s < -127 ? -127 : (s > 127 ? 127 : s);
      sbyte = (uint8_t)(s + 127);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        out[i] = e4m3x4(ldexpf(bf16_to_f32(d[2 * i] & 0xffffu), -s), ldexpf(bf16_to_f32(d[2 * i] >> 16), -s),
                        ldexpf(bf16_to_f32(d[2 * i + 1] & 0xffffu), -s), ldexpf(bf16_to_f32(d[2 * i + 1] >> 16), -s));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = 0;
    }
    uint4* dst = reinterpret_cast<uint4*>(q + b * 32);
    dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
    dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
    sc[b] = sbyte;
  }
}

hipError_t launch_mx_quantize(const uint16_t* x, long rows, int K, uint8_t* q, uint8_t* sc, hipStream_t s) {
  long nb = rows * (K / 32);
  hipLaunchKernelGGL(k_mx_quantize, dim3(grid_for(nb, 256, 16384)), dim3(256), 0, s, x, nb, q, sc);
  return hipGetLastError();
}

}  // namespace moe
