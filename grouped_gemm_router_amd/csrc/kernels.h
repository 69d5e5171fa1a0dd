// Host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Arguments of every grouped GEMM of the layer (unused fields stay null).
struct GemmArgs {
  int T, H, I, E, k;
  int act;                // gated activation (moe_activation)
  float act_limit;        // its clamp, where it has one
  const int32_t* offsets;
  const int32_t* row_token;
  const int32_t* row_slot;
  const float* topk_w;
  const uint16_t* X;
  const uint16_t* dY;
  const uint16_t* Wg_t;   // [E, I, H]
  const uint16_t* Wu_t;   // [E, I, H]
  const uint16_t* Wd_t;   // [E, H, I]
  uint16_t* Hrows;        // [A, I]  h (forward)
  uint16_t* Orows;        // [A, H]
  uint16_t* hw;           // [A, I]  bf16(w h) (backward; w = the row's top-k weight)
  uint16_t* hw_lo;        // [A, I]  bf16 of its remainder, w h - bf16(w h)
  float* P;               // [A, I]
  uint16_t* dGU;          // [A, 2I]  bf16(dg) | bf16(du)
  uint16_t* dGU_lo;       // [A, 2I]  bf16 of the remainders (dg - bf16(dg), du - bf16(du))
  float* dXr;             // [A, H]
  float* dwt_part;        // [A, nparts]
  int nparts;
  float* GU;              // [A, 2I] fp32: G in columns [0, I), U in [I, 2I) (saved-activation path:
                          // written by the forward gate/up GEMM when set, read by the backward)
  uint16_t* dWg;
  uint16_t* dWu;
  uint16_t* dWd;
  int32_t* wlist;         // small-token path: work list in the workspace
};

int num_cus();

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* idx, float* w,
                        hipStream_t s);
hipError_t launch_route_backward(const int32_t* idx, const float* w, const float* dw, int T, int E, int k,
                                 float* dl, hipStream_t s);
size_t dispatch_ws_bytes(long A, int E);
// dispatch of T*k <= DISPATCH_SMALL_A slots runs in one workgroup
constexpr int DISPATCH_SMALL_A = 4096;
hipError_t launch_dispatch(const int32_t* idx, int T, int E, int k, int32_t* offsets,
                           int32_t* row_token, int32_t* row_slot, int32_t* slot_row,
                           int32_t* ws, hipStream_t s);
hipError_t launch_pack(const uint16_t* W, int E, int K, int N, uint16_t* Wt, hipStream_t s);
hipError_t launch_mx_quantize(const uint16_t* x, long rows, int K, uint8_t* q, uint8_t* sc,
                              hipStream_t s);
hipError_t launch_combine(const uint16_t* O, const int32_t* slot_row, const float* w, int T,
                          int k, int H, uint16_t* Y, hipStream_t s);

// bf16 expert GEMMs
hipError_t launch_fwd_gateup(const GemmArgs& a, hipStream_t s);
hipError_t launch_fwd_down(const GemmArgs& a, hipStream_t s);
hipError_t launch_bwd_p(const GemmArgs& a, hipStream_t s);
hipError_t launch_bwd_recompute(const GemmArgs& a, hipStream_t s);
// the saved-activation backward's elementwise pass over P, G and U (in place of the recompute);
// its router-weight partial sums are one per row
hipError_t launch_bwd_act_rows(const GemmArgs& a, hipStream_t s);
hipError_t launch_bwd_dx_rows(const GemmArgs& a, hipStream_t s);
hipError_t launch_bwd_dw_down(const GemmArgs& a, hipStream_t s);
hipError_t launch_bwd_dw_gateup(const GemmArgs& a, hipStream_t s);
// router-weight partial sums per row of the recompute (its column tiles times waves across)
int bwd_nparts(int I, int act);
hipError_t launch_bwd_token_reduce(const GemmArgs& a, const int32_t* slot_row, uint16_t* dX,
                                   float* d_topk_w, hipStream_t s);

// small-token path: every expert has at most T <= DECODE_MAX_T rows
constexpr int DECODE_MAX_T = 64;
// workspace of the small-token path: the (expert, row group) work list
size_t decode_ws_bytes(int E);
hipError_t launch_decode_mlp(const GemmArgs& a, hipStream_t s);

// MXFP8 expert GEMMs
struct MxArgs {
  int T, H, I, E, k;
  int act;
  float act_limit;
  const int32_t* offsets;
  const int32_t* row_token;
  const uint8_t* Xq;  const uint8_t* Xs;    // [T, H], [T, H/32]
  const uint8_t* Wg;  const uint8_t* Sg;    // [E, I, H], [E, I, H/32]
  const uint8_t* Wu;  const uint8_t* Su;
  const uint8_t* Wd;  const uint8_t* Sd;    // [E, H, I], [E, H, I/32]
  uint16_t* Hrows;                          // [A, I] bf16
  const uint8_t* Hq;  const uint8_t* Hs;    // [A, I], [A, I/32]
  uint16_t* Orows;                          // [A, H]
  int stream_out;                           // store Orows non-temporally (it exceeds the last-level cache)
};
hipError_t launch_mx_gateup(const MxArgs& a, hipStream_t s);
hipError_t launch_mx_down(const MxArgs& a, hipStream_t s);

}  // namespace moe
