// MXFP8 grouped GEMMs (gate/up + SwiGLU, down) on gfx950's block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and one E8M0 scale per
// 32 contraction elements of every row (OCP Microscaling v1.0).
//
// Same persistent schedule, tile shape and LDS layout as the bf16 kernels: a
// 128-byte LDS row now holds 128 E4M3 codes (one k-tile), next to one 32-bit
// word per row holding the row's four scale bytes of that k-tile.
//
// Operand layout of the scaled MFMA (verified on the device): for a 64-long
// k chunk, lane half h (= lane / 32) supplies bytes [16h, 16h+16) and
// [32+16h, 32+16h+16) of its row, and its scale operand applies to the
// 32-element block [32h, 32h+32).  So MFMA kk of a k-tile reads 16-byte chunks
// 4kk+h and 4kk+2+h and scale byte 2kk+h.
#include "grouped_gemm.h"
#include "kernels.h"

namespace moe {

using CfgMx = TileCfg<256, 256, 2, 2>;
constexpr int BKB = 128;                 // fp8 codes (bytes) per k-tile
constexpr uint32_t SCALE_ONE = 0x7f7f7f7fu;

// K-contiguous rows of E4M3 codes and their E8M0 scales.  Src::rows(p, t, row, data, scales)
// sets data (element k = 0 of the row) and scales (its first scale byte), or leaves them null
// for a row of zeros.
template <int ROWS, int NT, class Src>
struct KRowsMx {
  static constexpr int CHUNKS = ROWS * 8;
  static constexpr int PER = (CHUNKS + NT - 1) / NT;
  static constexpr int SPER = (ROWS + NT - 1) / NT;
  const uint8_t* ptr[PER];
  uint4 reg[PER];
  const uint8_t* sptr[SPER];
  uint32_t sreg[SPER];

  __device__ void init(const MxArgs& p, const Tile& tl) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      const uint8_t *d = nullptr, *s = nullptr;
      if (c < CHUNKS) Src::rows(p, tl, c >> 3, d, s);
      ptr[i] = d ? d + (c & 7) * 16 : nullptr;
    }
#pragma unroll
    for (int i = 0; i < SPER; ++i) {
      const int r = threadIdx.x + i * NT;
      const uint8_t *d = nullptr, *s = nullptr;
      if (r < ROWS) Src::rows(p, tl, r, d, s);
      sptr[i] = d ? s : nullptr;
    }
  }
  __device__ void load(int k0) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      reg[i] = ptr[i] ? *reinterpret_cast<const uint4*>(ptr[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < SPER; ++i)
      sreg[i] = sptr[i] ? *reinterpret_cast<const uint32_t*>(sptr[i] + k0 / 32) : SCALE_ONE;
  }
  __device__ void store(uint4* lds, uint32_t* lds_s) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = threadIdx.x + i * NT;
      if (c < CHUNKS) lds[lds_chunk(c >> 3, c & 7)] = reg[i];
    }
#pragma unroll
    for (int i = 0; i < SPER; ++i) {
      const int r = threadIdx.x + i * NT;
      if (r < ROWS) lds_s[r] = sreg[i];
    }
  }
};

struct SrcMxX {  // gathered token rows of the quantised X
  __device__ static void rows(const MxArgs& p, const Tile& t, int row, const uint8_t*& d, const uint8_t*& s) {
    const int r = t.m0 + row;
    if (r < t.m_end) {
      const size_t tok = (size_t)p.row_token[r];
      d = p.Xq + tok * p.H;
      s = p.Xs + tok * (p.H / 32);
    }
  }
};
template <class C>
struct SrcMxGateUpW {  // packed [E, I, H] gate / up codes, interleaved per wave column group
  __device__ static void rows(const MxArgs& p, const Tile& t, int rr, const uint8_t*& d, const uint8_t*& s) {
    constexpr int half = C::WTN / 2;
    const int g = rr / C::WTN, within = rr % C::WTN;
    const bool up = within >= half;
    const int col = t.nt * (C::BN / 2) + g * half + (within % half);
    if (col < p.I) {
      const size_t row = (size_t)t.e * p.I + col;
      d = (up ? p.Wu : p.Wg) + row * p.H;
      s = (up ? p.Su : p.Sg) + row * (p.H / 32);
    }
  }
};
struct SrcMxH {  // expert-major quantised h rows
  __device__ static void rows(const MxArgs& p, const Tile& t, int row, const uint8_t*& d, const uint8_t*& s) {
    const int r = t.m0 + row;
    if (r < t.m_end) {
      d = p.Hq + (size_t)r * p.I;
      s = p.Hs + (size_t)r * (p.I / 32);
    }
  }
};
struct SrcMxDownW {  // packed [E, H, I] down codes
  __device__ static void rows(const MxArgs& p, const Tile& t, int rr, const uint8_t*& d, const uint8_t*& s) {
    const int n = t.n0 + rr;
    if (n < p.H) {
      const size_t row = (size_t)t.e * p.H + n;
      d = p.Wd + row * p.I;
      s = p.Sd + row * (p.I / 32);
    }
  }
};

template <class C>
__device__ __forceinline__ void mma_ktile_mx(const uint4* As, const uint32_t* As_s, const uint4* Bs,
                                             const uint32_t* Bs_s, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                                             int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    i32x8 a[C::FM], b[C::FN];
    int sa[C::FM], sb[C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int row = wm * C::WTM + fm * 32 + (lane & 31);
      const uint4 lo = As[lds_chunk(row, 4 * kk + h)], hi = As[lds_chunk(row, 4 * kk + 2 + h)];
      a[fm] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sa[fm] = (int)((As_s[row] >> (8 * (2 * kk + h))) & 0xffu);
    }
#pragma unroll
    for (int fn = 0; fn < C::FN; ++fn) {
      const int row = wn * C::WTN + fn * 32 + (lane & 31);
      const uint4 lo = Bs[lds_chunk(row, 4 * kk + h)], hi = Bs[lds_chunk(row, 4 * kk + 2 + h)];
      b[fn] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      sb[fn] = (int)((Bs_s[row] >> (8 * (2 * kk + h))) & 0xffu);
    }
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[fn], a[fm], acc[fm][fn], 0, 0, 0, sb[fn],
                                                                     0, sa[fm]);
  }
}

// Shared body: RowGroups schedule over the expert rows, two-stage LDS ring.
template <class C, class SrcA, class SrcB, class Epi>
__device__ __forceinline__ void mx_gemm_body(const MxArgs& p, int N, int K) {
  __shared__ uint4 smem[2 * (C::LDS_A + C::LDS_B)];
  __shared__ uint32_t sscale[2 * (C::BM + C::BN)];
  __shared__ int sched_lds[1024 + 1 + C::NT / 64 + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  RowGroups<C::BM, C::BN, C::NT> sched;
  sched.init(p.offsets, p.E, N, K, sched_lds, sched_lds + 1025);
  XcdWalk walk;
  walk.init(sched.total);
  for (; walk.valid(); walk.next()) {
    const Tile tl = sched.tile(walk.t);
    KRowsMx<C::BM, C::NT, SrcA> al;
    KRowsMx<C::BN, C::NT, SrcB> bl;
    al.init(p, tl);
    bl.init(p, tl);
    const int nk = K / BKB;
    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[fm][fn][v] = 0.f;
    uint4* const As = smem;
    uint4* const Bs = smem + 2 * C::LDS_A;
    uint32_t* const As_s = sscale;
    uint32_t* const Bs_s = sscale + 2 * C::BM;
    al.load(0);
    bl.load(0);
    al.store(As, As_s);
    bl.store(Bs, Bs_s);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < nk) {
        al.load((kt + 1) * BKB);
        bl.load((kt + 1) * BKB);
      }
      mma_ktile_mx<C>(As + cur * C::LDS_A, As_s + cur * C::BM, Bs + cur * C::LDS_B, Bs_s + cur * C::BN, acc, wm,
                      wn, lane);
      if (kt + 1 < nk) {
        al.store(As + (cur ^ 1) * C::LDS_A, As_s + (cur ^ 1) * C::BM);
        bl.store(Bs + (cur ^ 1) * C::LDS_B, Bs_s + (cur ^ 1) * C::BN);
      }
      __syncthreads();
    }
    Epi::apply(p, tl, acc, wm, wn, lane);
  }
}

template <class C>
struct MxSwiGLUEpi {  // h = bf16(silu(G) * U) -> Hrows
  __device__ static void apply(const MxArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                               int lane) {
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

template <class C>
struct MxStoreOEpi {  // O = bf16(acc) -> Orows
  __device__ static void apply(const MxArgs& p, const Tile& t, f32x16 (&acc)[C::FM][C::FN], int wm, int wn,
                               int lane) {
#pragma unroll
    for (int fm = 0; fm < C::FM; ++fm) {
      const int r = t.m0 + Frag<C>::row(wm, fm, lane);
      if (r >= t.m_end) continue;
      uint16_t* out = p.Orows + (size_t)r * p.H;
#pragma unroll
      for (int fn = 0; fn < C::FN; ++fn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = t.n0 + Frag<C>::col(wn, fn, q, lane);
          if (n >= p.H) continue;
          store_bf16x4(out + n, acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1], acc[fm][fn][4 * q + 2],
                       acc[fm][fn][4 * q + 3]);
        }
    }
  }
};

__global__ void __launch_bounds__(CfgMx::NT) k_mx_gateup(const MxArgs p) {
  mx_gemm_body<CfgMx, SrcMxX, SrcMxGateUpW<CfgMx>, MxSwiGLUEpi<CfgMx>>(p, 2 * p.I, p.H);
}
__global__ void __launch_bounds__(CfgMx::NT) k_mx_down(const MxArgs p) {
  mx_gemm_body<CfgMx, SrcMxH, SrcMxDownW, MxStoreOEpi<CfgMx>>(p, p.H, p.I);
}

static int mx_grid(const MxArgs& a, int N) {
  long A = (long)a.T * a.k;
  long mt = A / CfgMx::BM + (a.E < A ? a.E : A) + 1;
  long tiles = mt * ((N + CfgMx::BN - 1) / CfgMx::BN);
  long cap = (long)num_cus();
  long g = tiles < cap ? tiles : cap;
  return (int)((g + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
}

hipError_t launch_mx_gateup(const MxArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_mx_gateup, dim3(mx_grid(a, 2 * a.I)), dim3(CfgMx::NT), 0, s, a);
  return hipGetLastError();
}
hipError_t launch_mx_down(const MxArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_mx_down, dim3(mx_grid(a, a.H)), dim3(CfgMx::NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
