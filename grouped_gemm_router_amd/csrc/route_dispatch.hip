// Router (softmax -> top-k -> renormalise) and expert-major dispatch
// (histogram, prefix scan, stable scatter) on gfx950.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Router: a group of LPT lanes per token (16, 32 or 64; a wave routes 64/LPT
// tokens).  Each lane keeps NPL logits (E <= LPT*NPL) in registers; k rounds
// of a group arg-max pick the experts in descending logit order, ties to the
// lowest index.  The weights are exp(l_j - l_max) over the chosen logits,
// normalised by their sum (softmax over E renormalised over k).
//
// The arg-max runs on 64-bit keys that order exactly like (logit, -index):
// high word = the fp32 logit mapped to an unsigned integer of the same order
// (-0.0 first turned into +0.0), low word = ~index.  Inside each 16-lane row
// the maximum key is spread with DPP lane permutations (no LDS round trip);
// wider groups combine their row maxima through readlane.  Each round's
// winner is uniform over the group, so every lane accumulates the softmax
// numerators and their sum in round order, with no cross-lane sum.
//
// Narrow groups cut the VALU work per token (the work of a round grows with
// NPL, less than linearly, while a wave serves 64/LPT tokens at once); small
// batches keep whole-wave groups, whose rounds are shorter.
// ---------------------------------------------------------------------------
constexpr int ROUTE_MAX_PER_LANE = 16;
constexpr int ROUTE_NARROW_MIN_T = 1024;   // batches from this size on use 16- or 32-lane groups

__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)(~e);
}
__device__ __forceinline__ float route_key_logit(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7fffffffu) : ~u;
  return __uint_as_float(u);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}

// Maximum key of each LPT-lane group (every lane of the group gets it).
template <int LPT>
__device__ __forceinline__ uint64_t group_max_key(uint64_t k, int lane) {
  k = max_u64(k, dpp_u64<0xb1>(k));    // quad_perm [1,0,3,2]: lane ^ 1
  k = max_u64(k, dpp_u64<0x4e>(k));    // quad_perm [2,3,0,1]: lane ^ 2
  k = max_u64(k, dpp_u64<0x141>(k));   // row_half_mirror: the other quad of each 8
  k = max_u64(k, dpp_u64<0x140>(k));   // row_mirror: the other half of each 16
  if constexpr (LPT == 16) {
    return k;
  } else {
    const uint64_t r0 = readlane_u64(k, 0), r1 = readlane_u64(k, 16);
    const uint64_t r2 = readlane_u64(k, 32), r3 = readlane_u64(k, 48);
    const uint64_t lo = max_u64(r0, r1), hi = max_u64(r2, r3);
    if constexpr (LPT == 32) return lane < 32 ? lo : hi;
    else return max_u64(lo, hi);
  }
}

// Routes the tokens of one wave: token t0 + lane / LPT with the lanes of its
// group; writes each token's k expert ids (descending logit) and renormalised
// weights.  Every lane loads all its logits at once (an index past E reads
// logit 0 and is masked); groups past T route token t0 and write nothing.
template <int LPT, int NPL>
__device__ __forceinline__ void route_tokens(const float* __restrict__ logits, int T, int E, int k, int t0,
                                             int lane, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  const int l = lane % LPT;
  const int t = t0 + lane / LPT;
  const bool valid = t < T;
  const float* row = logits + (size_t)(valid ? t : t0) * E;
  float v[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) v[i] = row[(l + LPT * i < E) ? l + LPT * i : 0];
  uint64_t key[NPL];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int e = l + LPT * i;
    key[i] = (e < E) ? route_key(v[i], e) : 0ull;       // 0 sorts below every real key
  }
  int my_e = 0;                                         // lane j < k of the group keeps the j-th choice
  float my_ex = 0.f, sum = 0.f, first = 0.f;
  for (int j = 0; j < k; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) best = max_u64(best, key[i]);
    const uint64_t top = group_max_key<LPT>(best, lane);
    const int e = (int)~(uint32_t)top;
#pragma unroll
    for (int i = 0; i < NPL; ++i)
      if (l + LPT * i == e) key[i] = 0ull;              // taken
    const float lg = route_key_logit(top);
    if (j == 0) first = lg;
    const float ex = expf(lg - first);
    sum += ex;
    if (l == j) {
      my_e = e;
      my_ex = ex;
    }
  }
  if (valid && l < k) {
    topk_idx[(size_t)t * k + l] = my_e;
    topk_w[(size_t)t * k + l] = my_ex / sum;
  }
}

// The smallest logits-per-lane count that holds E (the work of a round grows with it).
template <int LPT>
__device__ __forceinline__ void route_wave(const float* __restrict__ logits, int T, int E, int k, int t0, int lane,
                                           int32_t* __restrict__ idx, float* __restrict__ w) {
  if (E <= LPT) route_tokens<LPT, 1>(logits, T, E, k, t0, lane, idx, w);
  else if (E <= 2 * LPT) route_tokens<LPT, 2>(logits, T, E, k, t0, lane, idx, w);
  else if (E <= 4 * LPT) route_tokens<LPT, 4>(logits, T, E, k, t0, lane, idx, w);
  else if (E <= 8 * LPT) route_tokens<LPT, 8>(logits, T, E, k, t0, lane, idx, w);
  else route_tokens<LPT, ROUTE_MAX_PER_LANE>(logits, T, E, k, t0, lane, idx, w);
}

template <int LPT>
__global__ void __launch_bounds__(256) k_route(const float* __restrict__ logits, int T, int E, int k,
                                               int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  constexpr int TPW = 64 / LPT;                          // tokens per wave
  const int lane = threadIdx.x & 63;
  const int t0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW;
  if (t0 >= T) return;
  route_wave<LPT>(logits, T, E, k, t0, lane, topk_idx, topk_w);
}

// Group width: 16 lanes while E <= 256 and k <= 16, 32 while E <= 512 (k <= 32
// always), else 64; whole waves for batches under ROUTE_NARROW_MIN_T tokens.
static int route_group_lanes(int T, int E, int k) {
  if (T < ROUTE_NARROW_MIN_T || E > 32 * ROUTE_MAX_PER_LANE) return 64;
  if (E > 16 * ROUTE_MAX_PER_LANE || k > 16) return 32;
  return 16;
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w, hipStream_t s) {
  const int lpt = route_group_lanes(T, E, k);
  const int per_block = 4 * (64 / lpt);
  const dim3 grid((T + per_block - 1) / per_block);
  if (lpt == 16) hipLaunchKernelGGL(k_route<16>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
  else if (lpt == 32) hipLaunchKernelGGL(k_route<32>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
  else hipLaunchKernelGGL(k_route<64>, grid, dim3(256), 0, s, logits, T, E, k, idx, w);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Router backward (LightMoE "MoE training": router gradients).  On the chosen
// logits the weights are a softmax, so for e = topk_idx[t, j]
//   d_logits[t, e] = w_j (d_j - sum_i w_i d_i),
// and every other logit of the token gets 0.  One wave per token: lane j < k
// holds slot j; the sum runs over j in ascending order, the same in every lane;
// lane l writes the logits l, l + 64, ... once each (coalesced, no ordering
// between stores to one address needed).  Ids outside [0, E) are skipped.
// ---------------------------------------------------------------------------
template <int NPL>
__device__ __forceinline__ void route_backward_token(const int32_t* idx, const float* w, const float* dw, int E,
                                                     int k, int lane, float* out) {
  const int my = lane < k ? idx[lane] : -1;
  const float mw = lane < k ? w[lane] : 0.f, md = lane < k ? dw[lane] : 0.f;
  const float prod = mw * md;
  float s = 0.f;
  for (int j = 0; j < k; ++j) s += __shfl(prod, j, 64);
  const float g = mw * (md - s);
  float v[NPL];
#pragma unroll
  for (int p = 0; p < NPL; ++p) v[p] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int e = __shfl(my, j, 64);
    const float gj = __shfl(g, j, 64);
    if (e >= 0 && e < E && (e & 63) == lane) {
#pragma unroll
      for (int p = 0; p < NPL; ++p)
        if ((e >> 6) == p) v[p] = gj;
    }
  }
#pragma unroll
  for (int p = 0; p < NPL; ++p) {
    const int e = p * 64 + lane;
    if (e < E) out[e] = v[p];
  }
}

template <int NPL>
__global__ void __launch_bounds__(256) k_route_backward(const int32_t* __restrict__ idx, const float* __restrict__ w,
                                                        const float* __restrict__ dw, int T, int E, int k,
                                                        float* __restrict__ dl) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t o = (size_t)t * k;
  route_backward_token<NPL>(idx + o, w + o, dw + o, E, k, lane, dl + (size_t)t * E);
}

hipError_t launch_route_backward(const int32_t* idx, const float* w, const float* dw, int T, int E, int k,
                                 float* dl, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64) hipLaunchKernelGGL(k_route_backward<1>, grid, block, 0, s, idx, w, dw, T, E, k, dl);
  else if (E <= 128) hipLaunchKernelGGL(k_route_backward<2>, grid, block, 0, s, idx, w, dw, T, E, k, dl);
  else if (E <= 256) hipLaunchKernelGGL(k_route_backward<4>, grid, block, 0, s, idx, w, dw, T, E, k, dl);
  else if (E <= 512) hipLaunchKernelGGL(k_route_backward<8>, grid, block, 0, s, idx, w, dw, T, E, k, dl);
  else hipLaunchKernelGGL(k_route_backward<16>, grid, block, 0, s, idx, w, dw, T, E, k, dl);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dispatch.  The T*k slots are cut into chunks of DISPATCH_CHUNK (one block,
// four waves of DISPATCH_CHUNK / 4 consecutive slots each).  Inside a wave, 64 slots are handled
// at a time: ten ballots over the bits of the expert id give every lane the
// mask of lanes holding the same expert, so its rank among equal experts in
// slot order is a popcount, and one lane per expert updates the running count.
// No atomics anywhere: the positions are the same on every run.
//   k_dispatch_count:   per-wave histograms  -> ws[e * nsub + chunk*4 + wave]
//   k_dispatch_scatter: offsets (scan of the totals), per-wave bases, then the
//                       stable scatter of (row_token, row_slot, slot_row).
// ---------------------------------------------------------------------------
#ifndef MOE_DISPATCH_CHUNK
#define MOE_DISPATCH_CHUNK 2048
#endif
constexpr int DISPATCH_CHUNK = MOE_DISPATCH_CHUNK;
constexpr int DISPATCH_WAVE_SLOTS = DISPATCH_CHUNK / 4;
static_assert(DISPATCH_WAVE_SLOTS % 64 == 0, "whole groups of 64 slots per wave");
constexpr int DISPATCH_MAX_E = 1024;

size_t dispatch_ws_bytes(long A, int E) {
  long nchunks = (A + DISPATCH_CHUNK - 1) / DISPATCH_CHUNK;
  if (nchunks < 1) nchunks = 1;
  return (size_t)nchunks * 4 * E * sizeof(int32_t);
}

// Mask of the lanes whose 11-bit key equals this lane's key.
__device__ __forceinline__ uint64_t match_key(int key) {
  uint64_t m = ~0ull;
#pragma unroll
  for (int b = 0; b < 11; ++b) {
    uint64_t bal = __ballot((key >> b) & 1);
    m &= ((key >> b) & 1) ? bal : ~bal;
  }
  return m;
}

__global__ void __launch_bounds__(256) k_dispatch_count(const int32_t* __restrict__ idx, long A, int E,
                                                        int nsub, int32_t* __restrict__ counts) {
  __shared__ int hist[4][DISPATCH_MAX_E];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long base = (long)blockIdx.x * DISPATCH_CHUNK + wave * DISPATCH_WAVE_SLOTS;
  int ids[DISPATCH_WAVE_SLOTS / 64];          // all of this wave's ids in flight at once
#pragma unroll
  for (int g = 0; g < DISPATCH_WAVE_SLOTS / 64; ++g) {
    const long s = base + g * 64 + lane;
    ids[g] = (s < A) ? idx[s] : -1;
  }
  for (int e = threadIdx.x; e < E; e += 256) hist[0][e] = hist[1][e] = hist[2][e] = hist[3][e] = 0;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < DISPATCH_WAVE_SLOTS / 64; ++g) {
    int e = ids[g];
    if (e >= E) e = -1;                       // out-of-range ids are skipped
    int key = (e >= 0) ? e : 0x400;
    uint64_t m = match_key(key);
    // the highest lane of each group of equal experts adds the group size
    bool leader = (m >> lane) == 1ull;
    if (e >= 0 && leader) hist[wave][key] += __popcll(m);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    *reinterpret_cast<int4*>(counts + (long)e * nsub + blockIdx.x * 4) =
        make_int4(hist[0][e], hist[1][e], hist[2][e], hist[3][e]);
}

// Sums of an expert's per-wave counts, over the int4 groups q0, q0 + dq, ...
// below nq (one group per chunk): of all of them, and of those of chunks
// before `me`.  The counts of one expert are contiguous; sixteen int4 loads
// are in flight at a time.
__device__ __forceinline__ void expert_count_sums(const int4* __restrict__ c4, int q0, int nq, int dq, int me,
                                                  int& all, int& before) {
  all = 0;
  before = 0;
  int q = q0;
  for (; q + 15 * dq < nq; q += 16 * dq) {
    int4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = c4[q + i * dq];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int sq = v[i].x + v[i].y + v[i].z + v[i].w;
      all += sq;
      before += (q + i * dq < me) ? sq : 0;
    }
  }
  for (; q < nq; q += dq) {
    const int4 v = c4[q];
    const int sq = v.x + v.y + v.z + v.w;
    all += sq;
    before += (q < me) ? sq : 0;
  }
}

// Threads per expert in the scatter's count sums: the largest power of two
// (at most 64, so a group stays inside one wave) with E * P <= 256, else 1.
__device__ __forceinline__ int count_parts(int E) {
  int P = 1;
  while (P < 64 && 2 * P * E <= 256) P *= 2;
  return P;
}

__global__ void __launch_bounds__(256) k_dispatch_scatter(const int32_t* __restrict__ idx, long A, int E, int k,
                                                          const int32_t* __restrict__ counts, int nsub,
                                                          int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_token,
                                                          int32_t* __restrict__ row_slot,
                                                          int32_t* __restrict__ slot_row) {
  __shared__ int base[4][DISPATCH_MAX_E];
  __shared__ int total[DISPATCH_MAX_E];
  __shared__ int red[8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int me = (int)blockIdx.x;
  // this wave's ids first: their loads overlap the count sums below
  const long sbase = (long)blockIdx.x * DISPATCH_CHUNK + wave * DISPATCH_WAVE_SLOTS;
  int ids[DISPATCH_WAVE_SLOTS / 64];
#pragma unroll
  for (int g = 0; g < DISPATCH_WAVE_SLOTS / 64; ++g) {
    const long s = sbase + g * 64 + lane;
    ids[g] = (s < A) ? idx[s] : -1;
  }
  // per expert (P threads each, summing every P-th chunk): its total, and per
  // wave of this chunk the number of its slots in earlier chunks and earlier
  // waves (relative to the expert's offset)
  const int P = count_parts(E);
  for (int e = threadIdx.x / P; e < E; e += 256 / P) {
    const int4* c4 = reinterpret_cast<const int4*>(counts + (long)e * nsub);
    const int4 mine = c4[me];
    int all, before;
    expert_count_sums(c4, (int)threadIdx.x % P, nsub / 4, P, me, all, before);
    for (int o = 1; o < P; o <<= 1) {          // the P threads of an expert are adjacent lanes
      all += __shfl_xor(all, o, 64);
      before += __shfl_xor(before, o, 64);
    }
    if ((int)threadIdx.x % P == 0) {
      total[e] = all;
      base[0][e] = before;
      base[1][e] = before + mine.x;
      base[2][e] = before + mine.x + mine.y;
      base[3][e] = before + mine.x + mine.y + mine.z;
    }
  }
  __syncthreads();
  // exclusive scan of the totals over experts (4 consecutive experts per thread)
  int tot[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = threadIdx.x * 4 + i;
    tot[i] = (e < E) ? total[e] : 0;
    sum += tot[i];
  }
  int x = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int wave_base = 0;
  for (int w = 0; w < wave; ++w) wave_base += red[w];
  int ex = wave_base + x - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = threadIdx.x * 4 + i;
    if (e < E) {
      if (blockIdx.x == 0) offsets[e] = ex;
#pragma unroll
      for (int w = 0; w < 4; ++w) base[w][e] += ex;
    }
    ex += tot[i];
  }
  if (blockIdx.x == 0 && threadIdx.x == 255) offsets[E] = ex;
  __syncthreads();
  // stable scatter of this wave's slots
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int g = 0; g < DISPATCH_WAVE_SLOTS / 64; ++g) {
    long s = sbase + g * 64 + lane;
    int e = ids[g];
    if (e >= E) e = -1;                       // out-of-range ids are skipped
    int key = (e >= 0) ? e : 0x400;
    uint64_t m = match_key(key);
    if (e >= 0) {
      int pos = base[wave][key] + __popcll(m & below);
      row_token[pos] = (int)(s / k);
      row_slot[pos] = (int)s;
      slot_row[s] = pos;
    } else if (s < A) {
      slot_row[s] = -1;                       // a skipped slot has no row
    }
    // wave-wide order: all lanes read base before the leaders update it
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && (m >> lane) == 1ull) base[wave][key] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// Dispatch of a small batch (T*k <= DISPATCH_SMALL_A) in one workgroup of 16
// waves and one launch: the same histogram / scan / stable scatter as
// k_dispatch_count + k_dispatch_scatter, with each wave owning a contiguous
// run of slots (NG groups of 64 at most) and its histogram row in LDS.  The
// launch takes the smallest NG that holds the batch: every group is unrolled,
// and the unused ones cost about as much as the used (a decode batch of 256
// slots: 7.3 us with four groups per wave, 4.5 us with one).
// ---------------------------------------------------------------------------
constexpr int DS_WAVES = 16;

template <int NG>
__global__ void __launch_bounds__(64 * DS_WAVES) k_dispatch_small(
    const int32_t* __restrict__ idx, int A, int E, int k, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_slot, int32_t* __restrict__ slot_row) {
  static_assert(NG * 64 * DS_WAVES <= DISPATCH_SMALL_A, "groups per wave");
  __shared__ int hist[DS_WAVES][DISPATCH_MAX_E];
  __shared__ int red[DS_WAVES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int per = ((A + DS_WAVES - 1) / DS_WAVES + 63) / 64 * 64;     // slots per wave, whole groups of 64
  const int s0 = wave * per;
  int ids[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int s = s0 + g * 64 + lane;
    int e = (g * 64 < per && s < A) ? idx[s] : -1;
    ids[g] = (e >= 0 && e < E) ? e : 0x400;                           // out-of-range ids are skipped
  }
  for (int e = threadIdx.x; e < E; e += 64 * DS_WAVES)                // only the columns of real experts
#pragma unroll
    for (int w = 0; w < DS_WAVES; ++w) hist[w][e] = 0;
  __syncthreads();
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int key = ids[g];
    const uint64_t m = match_key(key);
    if (key < 0x400 && (m >> lane) == 1ull) hist[wave][key] += __popcll(m);
  }
  __syncthreads();
  // thread e: total of expert e, exclusive scan over experts, per-wave bases (the
  // expert's DS_WAVES counts are read once into registers)
  const int e = threadIdx.x;
  int cnt[DS_WAVES];
  int tot = 0;
#pragma unroll
  for (int w = 0; w < DS_WAVES; ++w) {
    cnt[w] = (e < E) ? hist[w][e] : 0;
    tot += cnt[w];
  }
  int x = tot;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int ex = x - tot;
  for (int w = 0; w < wave; ++w) ex += red[w];
  if (e < E) {
    offsets[e] = ex;
    if (e == E - 1) offsets[E] = ex + tot;
    int run = ex;
#pragma unroll
    for (int w = 0; w < DS_WAVES; ++w) {
      hist[w][e] = run;
      run += cnt[w];
    }
  }
  __syncthreads();
  // stable scatter of this wave's slots
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int s = s0 + g * 64 + lane;
    const int key = ids[g];
    const uint64_t m = match_key(key);
    if (key < 0x400) {
      const int pos = hist[wave][key] + __popcll(m & below);
      row_token[pos] = s / k;
      row_slot[pos] = s;
      slot_row[s] = pos;
    } else if (g * 64 < per && s < A) {
      slot_row[s] = -1;                       // a skipped slot has no row
    }
    __builtin_amdgcn_wave_barrier();
    if (key < 0x400 && (m >> lane) == 1ull) hist[wave][key] += __popcll(m);
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_dispatch(const int32_t* idx, int T, int E, int k, int32_t* offsets, int32_t* row_token,
                           int32_t* row_slot, int32_t* slot_row, int32_t* ws, hipStream_t s) {
  long A = (long)T * k;
  if (A > 0 && A <= DISPATCH_SMALL_A) {
    auto kern = A <= 64 * DS_WAVES ? k_dispatch_small<1> : A <= 128 * DS_WAVES ? k_dispatch_small<2>
                                                                                : k_dispatch_small<4>;
    hipLaunchKernelGGL(kern, dim3(1), dim3(64 * DS_WAVES), 0, s, idx, (int)A, E, k, offsets, row_token, row_slot,
                       slot_row);
    return hipGetLastError();
  }
  int nchunks = (int)((A + DISPATCH_CHUNK - 1) / DISPATCH_CHUNK);
  if (nchunks < 1) nchunks = 1;  // block 0 still writes the offsets when there are no slots
  hipLaunchKernelGGL(k_dispatch_count, dim3(nchunks), dim3(256), 0, s, idx, A, E, nchunks * 4, ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(k_dispatch_scatter, dim3(nchunks), dim3(256), 0, s, idx, A, E, k, ws, nchunks * 4,
                     offsets, row_token, row_slot, slot_row);
  return hipGetLastError();
}

}  // namespace moe
