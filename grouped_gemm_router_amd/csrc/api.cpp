// C ABI of the MoE layer (include/moe.h): argument checks on the host before
// any launch, workspace sizing, the gfx950 device check, and the launches.
#include "moe.h"

#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr int MAX_E = 1024;
constexpr int MAX_K = 32;
constexpr size_t ALIGN = 256;
// MI355X's last-level (Infinity) cache.  The MXFP8 down projection's output rows are stored
// non-temporally when they exceed it: the combine then finds few of them cached either way, and
// the streamed stores leave L2 to the row and weight tiles the GEMM re-reads.
constexpr size_t LAST_LEVEL_CACHE_BYTES = (size_t)256 << 20;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_route_args(int32_t T, int32_t E, int32_t k) {
  if (T < 0 || E < 1 || k < 1) return MOE_ERR_INVALID_ARG;
  if (k > E) return MOE_ERR_INVALID_ARG;
  if (E > MAX_E || k > MAX_K) return MOE_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)T * k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

moe_status check_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  moe_status s = check_route_args(p->T, p->E, p->k);
  if (s != MOE_OK) return s;
  if (p->H < 1 || p->I < 1) return MOE_ERR_INVALID_ARG;
  if (p->dtype != MOE_DTYPE_BF16 && p->dtype != MOE_DTYPE_MXFP8) return MOE_ERR_INVALID_ARG;
  if (p->activation < MOE_ACT_SWIGLU || p->activation > MOE_ACT_RELU2) return MOE_ERR_INVALID_ARG;
  if ((p->activation == MOE_ACT_SWIGLU_CLAMP || p->activation == MOE_ACT_SWIGLU_OAI) &&
      !(p->act_limit > 0.f && p->act_limit < 3.0e38f))
    return MOE_ERR_INVALID_ARG;
  const int align = p->dtype == MOE_DTYPE_MXFP8 ? 128 : 64;
  if (p->H % align || p->I % align) return MOE_ERR_UNSUPPORTED_SHAPE;
  // the row loaders use 32-bit byte offsets: token rows (X, dY: T*H bf16) and expert-major
  // rows (up to 2I bf16 each: dg|du) must stay below 4 GiB
  if ((int64_t)p->T * p->H >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)p->T * p->k * (int64_t)p->I >= (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED_SHAPE;
  return MOE_OK;
}

size_t mlp_ws(const moe_problem* p) {
  if (p->dtype != MOE_DTYPE_MXFP8) return p->T <= moe::DECODE_MAX_T ? align_up(moe::decode_ws_bytes(p->E)) : 0;
  const size_t T = p->T, H = p->H, I = p->I, A = (size_t)p->T * p->k;
  return align_up(T * H) + align_up(T * H / 32) + align_up(A * I) + align_up(A * I / 32);
}

size_t bwd_ws(const moe_problem* p) {
  const size_t H = p->H, I = p->I, A = (size_t)p->T * p->k;
  const size_t nparts = moe::bwd_nparts(p->I, p->activation);
  return align_up(A * I * 4) + 2 * align_up(A * 2 * I * 2) + 2 * align_up(A * I * 2) + align_up(A * H * 4) +
         align_up(A * nparts * 4);
}

// Device check, cached per device id.
std::mutex g_mu;
int g_dev_state[64];   // 0 unknown, 1 gfx950, 2 other
int g_dev_cus[64];

moe_status device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_UNSUPPORTED_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_dev_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_ERR_HIP;
    g_dev_state[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_cus[dev] = prop.multiProcessorCount;
  }
  return g_dev_state[dev] == 1 ? MOE_OK : MOE_ERR_UNSUPPORTED_DEVICE;
}

// Workspace of moe_expert_mlp_static, for callers that cannot allocate: one array per GPU, held
// until the process ends.  On the host, `scratch` names a host-side stand-in, never the device
// array: its device address comes from hipGetSymbolAddress, once per device (g_scratch).
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];
void* g_scratch[64];

// The current device's address of `scratch` (looked up on the device's first call, under g_mu).
moe_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= 64) return MOE_ERR_UNSUPPORTED_DEVICE;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MOE_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

namespace moe {
int num_cus() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  int n = (dev >= 0 && dev < 64) ? g_dev_cus[dev] : 0;
  return n > 0 ? n : 256;
}
}  // namespace moe

extern "C" {

MOE_API const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED_SHAPE: return "MOE_ERR_UNSUPPORTED_SHAPE";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_UNSUPPORTED_DEVICE: return "MOE_ERR_UNSUPPORTED_DEVICE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

MOE_API moe_status moe_validate_problem(const moe_problem* p) { return check_problem(p); }

MOE_API moe_status moe_workspace_size(const moe_problem* p, int call, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  moe_status s = check_problem(p);
  if (s != MOE_OK) return s;
  switch (call) {
    case MOE_CALL_DISPATCH: *bytes = align_up(moe::dispatch_ws_bytes((long)p->T * p->k, p->E)); break;
    case MOE_CALL_EXPERT_MLP: *bytes = mlp_ws(p); break;
    case MOE_CALL_BACKWARD:
      if (p->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_SHAPE;
      *bytes = bwd_ws(p);
      break;
    default: return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

MOE_API moe_status moe_check_device(void) { return device_ok(); }

MOE_API moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k, int32_t* topk_idx,
                             float* topk_w, void* stream) {
  moe_status s = check_route_args(T, E, k);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;                            // empty batch: nothing to read or write
  if (!logits || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if ((s = device_ok()) != MOE_OK) return s;
  return from_hip(moe::launch_route(logits, T, E, k, topk_idx, topk_w, (hipStream_t)stream));
}

MOE_API moe_status moe_route_backward(const int32_t* topk_idx, const float* topk_w, const float* d_topk_w,
                                      int32_t T, int32_t E, int32_t k, float* d_logits, void* stream) {
  moe_status s = check_route_args(T, E, k);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;                            // empty batch: nothing to read or write
  if (!topk_idx || !topk_w || !d_topk_w || !d_logits) return MOE_ERR_INVALID_ARG;
  if ((s = device_ok()) != MOE_OK) return s;
  return from_hip(moe::launch_route_backward(topk_idx, topk_w, d_topk_w, T, E, k, d_logits, (hipStream_t)stream));
}

MOE_API moe_status moe_dispatch(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                                int32_t* expert_offsets, int32_t* row_token, int32_t* row_slot,
                                int32_t* slot_row, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_route_args(T, E, k);
  if (s != MOE_OK) return s;
  if (!expert_offsets || (T > 0 && (!topk_idx || !row_token || !row_slot || !slot_row)))
    return MOE_ERR_INVALID_ARG;
  const size_t need = moe::dispatch_ws_bytes((long)T * k, E);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if ((s = device_ok()) != MOE_OK) return s;
  return from_hip(moe::launch_dispatch(topk_idx, T, E, k, expert_offsets, row_token, row_slot, slot_row,
                                       (int32_t*)ws, (hipStream_t)stream));
}

MOE_API moe_status moe_pack_weights(const void* W, int32_t E, int32_t K, int32_t N, void* Wt, void* stream) {
  if (!W || !Wt || E < 1 || K < 1 || N < 1) return MOE_ERR_INVALID_ARG;
  if (K % 64 || N % 64 || E > 65535) return MOE_ERR_UNSUPPORTED_SHAPE;
  moe_status s = device_ok();
  if (s != MOE_OK) return s;
  return from_hip(moe::launch_pack((const uint16_t*)W, E, K, N, (uint16_t*)Wt, (hipStream_t)stream));
}

MOE_API moe_status moe_mx_quantize(const void* x, int64_t rows, int32_t K, uint8_t* q, uint8_t* scales,
                                   void* stream) {
  if (rows < 0 || K < 1) return MOE_ERR_INVALID_ARG;
  if (K % 32) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!x || !q || !scales) return MOE_ERR_INVALID_ARG;
  moe_status s = device_ok();
  if (s != MOE_OK) return s;
  return from_hip(moe::launch_mx_quantize((const uint16_t*)x, rows, K, q, scales, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// moe_expert_mlp, with the workspace given by the caller or (use_static) the library's static
// array of MOE_STATIC_SCRATCH_BYTES on the current device.
// With GU (bf16 only) the forward also writes the fp32 projections of every routed row, on the
// row-grouped GEMMs for every T.
moe_status expert_mlp(const moe_problem* p, const void* X, const int32_t* row_token, const int32_t* expert_offsets,
                      const void* Wg_t, const void* Wu_t, const void* Wd_t, const uint8_t* Sg, const uint8_t* Su,
                      const uint8_t* Sd, void* H_rows, void* O_rows, void* ws, size_t ws_bytes, bool use_static,
                      void* stream, float* GU = nullptr, bool save_gu = false) {
  moe_status s = check_problem(p);
  if (s != MOE_OK) return s;
  const bool gated = p->activation != MOE_ACT_RELU2;     // ReLU^2 experts have no gate weight
  const bool rows = p->T > 0;                            // token-sized arrays may be NULL for T = 0
  if (save_gu && p->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!expert_offsets || (gated && !Wg_t) || !Wu_t || !Wd_t) return MOE_ERR_INVALID_ARG;
  if (rows && (!X || !row_token || !H_rows || !O_rows || (save_gu && !GU))) return MOE_ERR_INVALID_ARG;
  const bool mx = p->dtype == MOE_DTYPE_MXFP8;
  if (mx != ((Sg || !gated) && Su && Sd)) return MOE_ERR_INVALID_ARG;
  if (!mx && (Sg || Su || Sd)) return MOE_ERR_INVALID_ARG;
  if (!rows) return MOE_OK;                              // empty batch: nothing to compute
  const size_t need = save_gu ? 0 : mlp_ws(p);
  if (use_static) {
    if (need > MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
    ws_bytes = MOE_STATIC_SCRATCH_BYTES;
  } else if (need && (!ws || ws_bytes < need)) {
    return MOE_ERR_WORKSPACE;
  }
  if ((s = device_ok()) != MOE_OK) return s;
  if (use_static && (s = static_scratch(&ws)) != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (!mx) {
    moe::GemmArgs a = {};
    a.T = p->T; a.H = p->H; a.I = p->I; a.E = p->E; a.k = p->k;
    a.act = p->activation; a.act_limit = p->act_limit;
    a.offsets = expert_offsets;
    a.row_token = row_token;
    a.X = (const uint16_t*)X;
    a.Wg_t = (const uint16_t*)Wg_t;
    a.Wu_t = (const uint16_t*)Wu_t;
    a.Wd_t = (const uint16_t*)Wd_t;
    a.Hrows = (uint16_t*)H_rows;
    a.Orows = (uint16_t*)O_rows;
    a.wlist = (int32_t*)ws;
    a.GU = save_gu ? GU : nullptr;
    if (!save_gu && p->T <= moe::DECODE_MAX_T) return from_hip(moe::launch_decode_mlp(a, st));
    hipError_t e = moe::launch_fwd_gateup(a, st);
    if (e == hipSuccess) e = moe::launch_fwd_down(a, st);
    return from_hip(e);
  }
  const size_t T = p->T, H = p->H, I = p->I, A = (size_t)p->T * p->k;
  uint8_t* w8 = (uint8_t*)ws;
  uint8_t* Xq = w8;
  uint8_t* Xs = Xq + align_up(T * H);
  uint8_t* Hq = Xs + align_up(T * H / 32);
  uint8_t* Hs = Hq + align_up(A * I);
  moe::MxArgs m = {};
  m.T = p->T; m.H = p->H; m.I = p->I; m.E = p->E; m.k = p->k;
  m.act = p->activation; m.act_limit = p->act_limit;
  m.offsets = expert_offsets;
  m.row_token = row_token;
  m.Xq = Xq; m.Xs = Xs;
  m.Wg = (const uint8_t*)Wg_t; m.Sg = Sg;
  m.Wu = (const uint8_t*)Wu_t; m.Su = Su;
  m.Wd = (const uint8_t*)Wd_t; m.Sd = Sd;
  m.Hrows = (uint16_t*)H_rows;
  m.Hq = Hq; m.Hs = Hs;
  m.Orows = (uint16_t*)O_rows;
  m.stream_out = A * H * 2 > LAST_LEVEL_CACHE_BYTES;
  hipError_t e = moe::launch_mx_quantize((const uint16_t*)X, p->T, p->H, Xq, Xs, st);
  if (e == hipSuccess) e = moe::launch_mx_gateup(m, st);
  if (e == hipSuccess) e = moe::launch_mx_quantize((const uint16_t*)H_rows, (long)A, p->I, Hq, Hs, st);
  if (e == hipSuccess) e = moe::launch_mx_down(m, st);
  return from_hip(e);
}

}  // namespace

extern "C" {

MOE_API moe_status moe_expert_mlp(const moe_problem* p, const void* X, const int32_t* row_token,
                                  const int32_t* expert_offsets, const void* Wg_t, const void* Wu_t,
                                  const void* Wd_t, const uint8_t* Sg, const uint8_t* Su, const uint8_t* Sd,
                                  void* H_rows, void* O_rows, void* ws, size_t ws_bytes, void* stream) {
  return expert_mlp(p, X, row_token, expert_offsets, Wg_t, Wu_t, Wd_t, Sg, Su, Sd, H_rows, O_rows, ws, ws_bytes,
                    false, stream);
}

MOE_API moe_status moe_expert_mlp_static(const moe_problem* p, const void* X, const int32_t* row_token,
                                         const int32_t* expert_offsets, const void* Wg_t, const void* Wu_t,
                                         const void* Wd_t, const uint8_t* Sg, const uint8_t* Su, const uint8_t* Sd,
                                         void* H_rows, void* O_rows, void* stream) {
  return expert_mlp(p, X, row_token, expert_offsets, Wg_t, Wu_t, Wd_t, Sg, Su, Sd, H_rows, O_rows, nullptr, 0,
                    true, stream);
}

MOE_API moe_status moe_expert_mlp_save(const moe_problem* p, const void* X, const int32_t* row_token,
                                       const int32_t* expert_offsets, const void* Wg_t, const void* Wu_t,
                                       const void* Wd_t, void* H_rows, void* O_rows, float* GU_rows, void* stream) {
  return expert_mlp(p, X, row_token, expert_offsets, Wg_t, Wu_t, Wd_t, nullptr, nullptr, nullptr, H_rows, O_rows,
                    nullptr, 0, false, stream, GU_rows, true);
}

MOE_API moe_status moe_grouped_gemm(int32_t dtype, const int32_t* m_indptr, int32_t E, int64_t M, int32_t N,
                                    int32_t K, const void* A, const uint8_t* SA, const void* B_t, const uint8_t* SB,
                                    void* C, void* stream) {
  if (dtype != MOE_DTYPE_BF16 && dtype != MOE_DTYPE_MXFP8) return MOE_ERR_INVALID_ARG;
  if (E < 1 || M < 0 || N < 1 || K < 1) return MOE_ERR_INVALID_ARG;
  const bool mx = dtype == MOE_DTYPE_MXFP8;
  const int align = mx ? 128 : 64;
  if (E > MAX_E || N % align || K % align) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (M >= ((int64_t)1 << 31) || M * K >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (!m_indptr || !B_t) return MOE_ERR_INVALID_ARG;
  if (M > 0 && (!A || !C)) return MOE_ERR_INVALID_ARG;
  if (mx != (SA && SB)) return MOE_ERR_INVALID_ARG;
  if (!mx && (SA || SB)) return MOE_ERR_INVALID_ARG;
  if (M == 0) return MOE_OK;                            // nothing to compute
  moe_status s = device_ok();
  if (s != MOE_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (!mx) {
    // the down projection's kernel: rows of A ("h", K = I) times B_t ([E, N = H, K]) into C
    moe::GemmArgs a = {};
    a.T = (int)M; a.k = 1; a.H = N; a.I = K; a.E = E;
    a.act = MOE_ACT_SWIGLU;
    a.offsets = m_indptr;
    a.Hrows = (uint16_t*)A;
    a.Wd_t = (const uint16_t*)B_t;
    a.Orows = (uint16_t*)C;
    return from_hip(moe::launch_fwd_down(a, st));
  }
  moe::MxArgs m = {};
  m.T = (int)M; m.k = 1; m.H = N; m.I = K; m.E = E;
  m.act = MOE_ACT_SWIGLU;
  m.offsets = m_indptr;
  m.Hq = (const uint8_t*)A; m.Hs = SA;
  m.Wd = (const uint8_t*)B_t; m.Sd = SB;
  m.Orows = (uint16_t*)C;
  m.stream_out = (size_t)M * N * 2 > LAST_LEVEL_CACHE_BYTES;
  return from_hip(moe::launch_mx_down(m, st));
}

MOE_API moe_status moe_combine(const void* O_rows, const int32_t* slot_row, const float* topk_w, int32_t T,
                               int32_t k, int32_t H, void* Y, void* stream) {
  if (T < 0 || k < 1 || k > MAX_K || H < 1) return MOE_ERR_INVALID_ARG;
  if (H % 8) return MOE_ERR_UNSUPPORTED_SHAPE;
  if ((int64_t)T * k >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED_SHAPE;
  if (T == 0) return MOE_OK;
  if (!O_rows || !slot_row || !topk_w || !Y) return MOE_ERR_INVALID_ARG;
  moe_status s = device_ok();
  if (s != MOE_OK) return s;
  return from_hip(moe::launch_combine((const uint16_t*)O_rows, slot_row, topk_w, T, k, H, (uint16_t*)Y,
                                      (hipStream_t)stream));
}

}  // extern "C"

namespace {

// moe_backward; with save_gu, G and U come from GU (moe_expert_mlp_save) and an elementwise pass
// over P, G and U replaces the recompute GEMM.
moe_status backward(const moe_problem* p, const void* X, const void* dY, const float* topk_w,
                    const int32_t* row_token, const int32_t* row_slot, const int32_t* slot_row,
                    const int32_t* expert_offsets, const void* Wg_t, const void* Wu_t, const void* Wd_t,
                    const float* GU, bool save_gu, void* dX, void* dW_gate, void* dW_up, void* dW_down,
                    float* d_topk_w, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_problem(p);
  if (s != MOE_OK) return s;
  if (p->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED_SHAPE;
  const bool gated = p->activation != MOE_ACT_RELU2;     // ReLU^2 experts have no gate weight
  const bool rows = p->T > 0;                            // token-sized arrays may be NULL for T = 0
  if (!expert_offsets || (gated && !Wg_t) || !Wu_t || !Wd_t || (gated && !dW_gate) || !dW_up || !dW_down)
    return MOE_ERR_INVALID_ARG;
  if (rows && (!X || !dY || !topk_w || !row_token || !row_slot || !slot_row || !dX || !d_topk_w))
    return MOE_ERR_INVALID_ARG;
  if (rows && save_gu && !GU) return MOE_ERR_INVALID_ARG;
  const size_t need = bwd_ws(p);
  if (need && (!ws || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  if ((s = device_ok()) != MOE_OK) return s;
  const size_t H = p->H, I = p->I, A = (size_t)p->T * p->k;
  uint8_t* w8 = (uint8_t*)ws;
  moe::GemmArgs a = {};
  a.T = p->T; a.H = p->H; a.I = p->I; a.E = p->E; a.k = p->k;
  a.act = p->activation; a.act_limit = p->act_limit;
  a.offsets = expert_offsets;
  a.row_token = row_token;
  a.row_slot = row_slot;
  a.topk_w = topk_w;
  a.X = (const uint16_t*)X;
  a.dY = (const uint16_t*)dY;
  a.Wg_t = (const uint16_t*)Wg_t;
  a.Wu_t = (const uint16_t*)Wu_t;
  a.Wd_t = (const uint16_t*)Wd_t;
  a.nparts = save_gu ? 1 : moe::bwd_nparts(p->I, p->activation);
  a.GU = const_cast<float*>(GU);
  a.P = (float*)w8;
  w8 += align_up(A * I * 4);
  a.dGU = (uint16_t*)w8;
  w8 += align_up(A * 2 * I * 2);
  a.dGU_lo = (uint16_t*)w8;
  w8 += align_up(A * 2 * I * 2);
  a.hw = (uint16_t*)w8;
  w8 += align_up(A * I * 2);
  a.hw_lo = (uint16_t*)w8;
  w8 += align_up(A * I * 2);
  a.dXr = (float*)w8;
  w8 += align_up(A * H * 4);
  a.dwt_part = (float*)w8;
  a.dWg = (uint16_t*)dW_gate;
  a.dWu = (uint16_t*)dW_up;
  a.dWd = (uint16_t*)dW_down;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (p->T > 0) {
    e = moe::launch_bwd_p(a, st);
    if (e == hipSuccess) e = save_gu ? moe::launch_bwd_act_rows(a, st) : moe::launch_bwd_recompute(a, st);
    if (e == hipSuccess) e = moe::launch_bwd_dx_rows(a, st);
    if (e == hipSuccess) e = moe::launch_bwd_token_reduce(a, slot_row, (uint16_t*)dX, d_topk_w, st);
  }
  if (e == hipSuccess) e = moe::launch_bwd_dw_down(a, st);
  if (e == hipSuccess) e = moe::launch_bwd_dw_gateup(a, st);
  return from_hip(e);
}

}  // namespace

extern "C" {

MOE_API moe_status moe_backward(const moe_problem* p, const void* X, const void* dY, const float* topk_w,
                                const int32_t* row_token, const int32_t* row_slot, const int32_t* slot_row,
                                const int32_t* expert_offsets, const void* Wg_t, const void* Wu_t,
                                const void* Wd_t, void* dX, void* dW_gate, void* dW_up, void* dW_down,
                                float* d_topk_w, void* ws, size_t ws_bytes, void* stream) {
  return backward(p, X, dY, topk_w, row_token, row_slot, slot_row, expert_offsets, Wg_t, Wu_t, Wd_t, nullptr, false,
                  dX, dW_gate, dW_up, dW_down, d_topk_w, ws, ws_bytes, stream);
}

MOE_API moe_status moe_backward_saved(const moe_problem* p, const void* X, const void* dY, const float* topk_w,
                                      const int32_t* row_token, const int32_t* row_slot, const int32_t* slot_row,
                                      const int32_t* expert_offsets, const void* Wg_t, const void* Wu_t,
                                      const void* Wd_t, const float* GU_rows, void* dX, void* dW_gate,
                                      void* dW_up, void* dW_down, float* d_topk_w, void* ws, size_t ws_bytes,
                                      void* stream) {
  return backward(p, X, dY, topk_w, row_token, row_slot, slot_row, expert_offsets, Wg_t, Wu_t, Wd_t, GU_rows, true,
                  dX, dW_gate, dW_up, dW_down, d_topk_w, ws, ws_bytes, stream);
}

}  // extern "C"
