/*
 * moe.h - C ABI of a routed Mixture-of-Experts expert layer for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer is the dropless top-k routed MoE described by the LigerCute
 * README ("LigerCute - native CUTLASS + NVSHMEM kernels": Overview, Forward
 * pass, Backward pass) and the LightMoE README (lightmoe 0.1.0: Grouped GEMM,
 * MoE inference, MoE training).  One GPU runs every expert:
 *
 *   moe_route       softmax over E logits -> top-k -> renormalise
 *   moe_dispatch    expert-major order of the T*k token-expert assignments
 *   moe_expert_mlp  grouped GEMM gate/up + activation, grouped GEMM down
 *   moe_combine     weighted sum of each token's k expert rows
 *   moe_backward    dX, dW_gate, dW_up, dW_down, d(top-k weights)
 *   moe_expert_mlp_save, moe_backward_saved  the training pair that keeps G, U
 *   moe_route_backward  d(router logits) from d(top-k weights)
 *   moe_grouped_gemm    standalone grouped GEMM over expert-major rows
 *
 * Conventions shared by every call
 * --------------------------------
 * - All tensor arguments are DEVICE pointers to dense row-major arrays; the
 *   shapes are given in elements next to each argument.  bf16 tensors are
 *   passed as raw 16-bit patterns.
 * - The caller owns every buffer: inputs, outputs and the workspace (sized by
 *   moe_workspace_size).  No call allocates device memory or synchronises;
 *   every call only enqueues work on `stream` (a hipStream_t, NULL for the
 *   default stream) and returns.  Use one workspace per concurrent stream.
 * - Arguments are checked on the host before anything is enqueued; on any
 *   error nothing is launched and the status says why.  A device that is not
 *   gfx950 gives MOE_ERR_UNSUPPORTED_DEVICE.  A launch failure gives
 *   MOE_ERR_HIP.  No C++ exception crosses this interface.
 * - Limits: 1 <= k <= min(E, 32); E <= 1024; T*k < 2^31; H and I multiples
 *   of 64 (MXFP8: multiples of 128); T*H < 2^31 and T*k*I < 2^30 (the row
 *   loaders address token rows and expert-major rows with 32-bit byte offsets).
 * - An empty batch (T = 0) is valid: every token-sized array (logits, X, dY,
 *   the routing and dispatch arrays, the row buffers, Y, dX, the top-k
 *   gradients) may then be NULL.  moe_dispatch still writes expert_offsets
 *   (all zero) and moe_backward still writes the weight gradients (zeros).
 * - Results are deterministic: the same inputs give bitwise-identical outputs
 *   (no floating-point atomics, fixed reduction orders).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,       /* null pointer, non-positive size, k > E ... */
  MOE_ERR_UNSUPPORTED_SHAPE = 2, /* outside the limits listed above */
  MOE_ERR_WORKSPACE = 3,         /* workspace missing or smaller than required */
  MOE_ERR_UNSUPPORTED_DEVICE = 4,/* current device is not gfx950 */
  MOE_ERR_HIP = 5                /* a HIP runtime call or launch failed */
} moe_status;

typedef enum {
  MOE_DTYPE_BF16 = 0,   /* X, weights and h in bf16 */
  MOE_DTYPE_MXFP8 = 1   /* X, weights and h as FP8 E4M3 with one E8M0 scale
                           per 32 elements along the contraction axis */
} moe_dtype;

/*
 * Activation h = f(G, U) of the expert MLP (G = x W_gate, U = x W_up).
 * LightMoE "Highlights" names SwiGLU-OAI, bounded SwiGLU, GeGLU, ReGLU and
 * ReLU^2 epilogues and "MoE inference" an activation clamp of 10 and ReLU^2
 * experts that load only an up and a down weight; the formulas are the public
 * definitions of the model families that use them.  ReLU^2 is ungated: the
 * expert has no W_gate, every gate pointer of a call may be NULL and is not
 * read, and dW_gate is not written.
 */
typedef enum {
  MOE_ACT_SWIGLU = 0,       /* silu(G) * U (the default) */
  MOE_ACT_SWIGLU_CLAMP = 1, /* silu(min(G, c)) * clamp(U, -c, c), c = act_limit (bounded SwiGLU) */
  MOE_ACT_SWIGLU_OAI = 2,   /* g * sigmoid(1.702 g) * (u + 1), g = min(G, c), u = clamp(U, -c, c) */
  MOE_ACT_GEGLU = 3,        /* gelu(G) * U, gelu(x) = x * Phi(x), Phi the normal CDF (erf form) */
  MOE_ACT_REGLU = 4,        /* max(G, 0) * U */
  MOE_ACT_RELU2 = 5         /* max(U, 0)^2 (no gate) */
} moe_activation;

/* Problem shape.  T tokens, hidden size H, expert intermediate size I,
 * E experts, k experts per token; the activation (a zeroed field is SwiGLU)
 * and the clamp c of the clamped ones (> 0, finite; ignored by the others). */
typedef struct {
  int32_t T, H, I, E, k;
  int32_t dtype;      /* moe_dtype */
  int32_t activation; /* moe_activation */
  float act_limit;    /* c of MOE_ACT_SWIGLU_CLAMP and MOE_ACT_SWIGLU_OAI */
} moe_problem;

/* Which call a workspace is sized for (moe_workspace_size). */
typedef enum {
  MOE_CALL_DISPATCH = 0,
  MOE_CALL_EXPERT_MLP = 1,
  MOE_CALL_BACKWARD = 2
} moe_call;

/* Human-readable name of a status code (static storage; host only). */
MOE_API const char* moe_status_string(int status);

/* Checks a problem against the limits above (host only, no device access). */
MOE_API moe_status moe_validate_problem(const moe_problem* p);

/* Bytes of device workspace `call` needs for problem `p` (host only). */
MOE_API moe_status moe_workspace_size(const moe_problem* p, int call, size_t* bytes);

/* MOE_OK when the current HIP device is gfx950 (queries the device once). */
MOE_API moe_status moe_check_device(void);

/*
 * Routing (LightMoE "MoE inference": top_k_ids int32 with distinct experts
 * per token, top_k_weights fp32; softmax -> top-k -> renormalise).
 *   logits   [T, E] fp32 in
 *   topk_idx [T, k] int32 out: experts in descending logit order, ties to the
 *            lowest expert index (-0.0 equals +0.0); NaN logits are invalid
 *   topk_w   [T, k] fp32 out: exp(l_j - l_max) / sum over the k chosen,
 *            equal to the softmax over all E renormalised over the k.
 */
MOE_API moe_status moe_route(const float* logits, int32_t T, int32_t E, int32_t k,
                             int32_t* topk_idx, float* topk_w, void* stream);

/*
 * Router backward (LightMoE "MoE training": deterministic router-gradient
 * kernels; the routing weights are made differentiable with respect to the
 * router output).  Gradient with respect to the logits of a loss whose gradient
 * with respect to the top-k weights of moe_route is d_topk_w.  On the chosen
 * logits the weights are a softmax, and the chosen set is piecewise constant,
 * so for e = topk_idx[t, j]:
 *   d_logits[t, e] = topk_w[t,j] * (d_topk_w[t,j] - sum_i topk_w[t,i] * d_topk_w[t,i])
 * (the sum in fp32 over i ascending), and every other element of row t is 0.
 *   topk_idx [T, k] int32, topk_w [T, k] fp32: as moe_route wrote them
 *            (ids outside [0, E) are skipped)
 *   d_topk_w [T, k] fp32 in (e.g. the d_topk_w of moe_backward)
 *   d_logits [T, E] fp32 out, every element written
 */
MOE_API moe_status moe_route_backward(const int32_t* topk_idx, const float* topk_w,
                                      const float* d_topk_w, int32_t T, int32_t E, int32_t k,
                                      float* d_logits, void* stream);

/*
 * Expert-major dispatch (LigerCute "Forward pass": routed tokens are sorted;
 * LightMoE "Grouped GEMM": contiguous expert-major rows with an int32
 * m_indptr of length E+1, zero-row experts valid; "MoE training": gather
 * indices and inverse slots).  Assignment (t, j) has slot s = t*k + j; rows
 * are grouped by expert and, inside an expert, ordered by slot.
 *   topk_idx       [T, k] int32 in, each value in [0, E), distinct per token
 *   expert_offsets [E+1] int32 out: rows of expert e are
 *                  [expert_offsets[e], expert_offsets[e+1])
 *   row_token      [T*k] int32 out: token of each row
 *   row_slot       [T*k] int32 out: slot of each row
 *   slot_row       [T*k] int32 out: row of each slot (inverse of row_slot)
 *   ws, ws_bytes   workspace of moe_workspace_size(MOE_CALL_DISPATCH)
 * An expert id outside [0, E) is skipped: its slot gets no row and
 * slot_row = -1, the rows of the valid slots keep their order, and
 * expert_offsets[E] counts the valid slots only (row_token and row_slot past
 * it are not written).  moe_combine and moe_backward give such a slot zero
 * contribution (and d_topk_w = 0), so no later call reads outside its buffers.
 * Ids repeated within a token are not detected: each copy gets its own row.
 */
MOE_API moe_status moe_dispatch(const int32_t* topk_idx, int32_t T, int32_t E, int32_t k,
                                int32_t* expert_offsets, int32_t* row_token,
                                int32_t* row_slot, int32_t* slot_row,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * Weight packing, done once when weights are loaded (LightMoE "Standalone
 * GEMM": packing is a separate operation, outside latency measurements; its
 * grouped GEMM takes b as [num_experts, N, K]).
 *   W  [E, K, N] bf16 in  (the math layout: x @ W)
 *   Wt [E, N, K] bf16 out (contraction axis contiguous)
 */
MOE_API moe_status moe_pack_weights(const void* W, int32_t E, int32_t K, int32_t N,
                                    void* Wt, void* stream);

/*
 * MXFP8 quantisation along rows (OCP Microscaling v1.0, section 6.3; the
 * per-32 E8M0 block scaling named by the cutedsl-megamoe page).  For every
 * block of 32 consecutive values: shared exponent = floor(log2(max|v|)) - 8
 * clamped to [-127, 127] (scale byte = exponent + 127; 0 for an all-zero
 * block); elements = v * 2^-exponent rounded to FP8 E4M3FN, to nearest even,
 * saturating at +-448.
 *   x      [rows, K] bf16 in, K a multiple of 32
 *   q      [rows, K] uint8 out (E4M3FN codes)
 *   scales [rows, K/32] uint8 out (E8M0)
 */
MOE_API moe_status moe_mx_quantize(const void* x, int64_t rows, int32_t K, uint8_t* q,
                                   uint8_t* scales, void* stream);

/*
 * Expert MLP over the expert-major rows (LightMoE "MoE inference": gate/up
 * projection, gated activation, requantisation, down projection):
 *   G = X[row_token[r]] W_gate[e], U = X[row_token[r]] W_up[e]   (fp32 accumulation)
 *   h[r] = bf16(f(G, U)) (f = p->activation, silu(G) * U by default),  O[r] = bf16(h[r] W_down[e])
 * for every row r of every expert e with rows.  Experts without rows are
 * never read.
 *   p              problem (dtype selects bf16 or MXFP8 operands)
 *   X              [T, H] bf16
 *   row_token, expert_offsets   from moe_dispatch
 *   bf16:  Wg_t, Wu_t [E, I, H] bf16 and Wd_t [E, H, I] bf16 (moe_pack_weights);
 *          Sg, Su, Sd must be NULL.  For MOE_ACT_RELU2, Wg_t (and Sg) may be NULL
 *   MXFP8: Wg_t, Wu_t [E, I, H] and Wd_t [E, H, I] E4M3 codes with
 *          Sg, Su [E, I, H/32] and Sd [E, H, I/32] E8M0 scales (moe_mx_quantize
 *          of the packed bf16 weights); X is quantised here, and h is
 *          requantised to MXFP8 along I before the down projection
 *   H_rows         [T*k, I] bf16 out (h, bf16 in both modes)
 *   O_rows         [T*k, H] bf16 out
 *   ws, ws_bytes   workspace of moe_workspace_size(MOE_CALL_EXPERT_MLP): the MXFP8
 *                  codes of X and h; for bf16 with T <= 64 a work list of 4E+1 int32
 *                  (bf16 with T > 64 needs none)
 */
MOE_API moe_status moe_expert_mlp(const moe_problem* p, const void* X, const int32_t* row_token,
                                  const int32_t* expert_offsets, const void* Wg_t,
                                  const void* Wu_t, const void* Wd_t, const uint8_t* Sg,
                                  const uint8_t* Su, const uint8_t* Sd, void* H_rows,
                                  void* O_rows, void* ws, size_t ws_bytes, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): moe_expert_mlp with its
 * workspace in a static device array of the library instead of a caller buffer.
 *   Arguments, results, kernels and error behaviour as moe_expert_mlp, without
 *   ws / ws_bytes.  The array holds MOE_STATIC_SCRATCH_BYTES on every GPU the
 *   library runs this call on, from the first call on that GPU until the process
 *   ends; a problem whose moe_workspace_size(MOE_CALL_EXPERT_MLP) exceeds it gives
 *   MOE_ERR_WORKSPACE before anything is enqueued (bf16 needs at most 16 KiB; MXFP8
 *   needs about T*H + T*k*I bytes).  The call allocates and frees nothing; its first
 *   call on a GPU looks up the array's device address (hipGetSymbolAddress).
 *   Every call on one GPU shares that GPU's array, which keeps the last call's
 *   contents (each call writes all it reads): calls that overlap on one GPU
 *   (other streams, other host threads) race and must be serialised by the caller.
 */
#define MOE_STATIC_SCRATCH_BYTES ((size_t)8 << 20)
MOE_API moe_status moe_expert_mlp_static(const moe_problem* p, const void* X,
                                         const int32_t* row_token, const int32_t* expert_offsets,
                                         const void* Wg_t, const void* Wu_t, const void* Wd_t,
                                         const uint8_t* Sg, const uint8_t* Su, const uint8_t* Sd,
                                         void* H_rows, void* O_rows, void* stream);

/*
 * Weighted combine (LigerCute "Forward pass": a final local combine applies
 * the router weights; LightMoE: routing-weight application and deterministic
 * combine):  Y[t] = bf16( sum_{j=0..k-1} topk_w[t,j] * O_rows[slot_row[t*k+j]] ),
 * accumulated in fp32 in ascending j.
 *   O_rows [T*k, H] bf16, slot_row [T*k] int32, topk_w [T, k] fp32, Y [T, H] bf16 out
 * slot_row must hold a row index in [0, T*k) or -1 (a slot moe_dispatch skipped,
 * which adds nothing), as moe_dispatch writes it.
 */
MOE_API moe_status moe_combine(const void* O_rows, const int32_t* slot_row, const float* topk_w,
                               int32_t T, int32_t k, int32_t H, void* Y, void* stream);

/*
 * Backward (LigerCute "Backward pass": activation recomputation, input and
 * expert-weight gradients, routed dX reduced back to the tokens; LightMoE:
 * deterministic input-, weight- and router-gradient kernels).  bf16 only.
 * Per row r (token t, slot s, expert e, weight w = topk_w[s]):
 *   G, U, h recomputed as in moe_expert_mlp;  P = dY[t] W_down[e]^T (fp32)
 *   d_topk_w[s] = <h, P>;  dh = w P
 *   du = dh * df/dU,  dg = dh * df/dG  (SwiGLU: du = dh * silu(G), dg = dh * U * silu'(G)),
 *   dO = w dY[t]   (P, dh, dg, du and dO are not rounded: the GEMMs that take dg, du and dO
 *                   as operands contract their bf16 value and their bf16 remainder)
 *   dX[t]      = bf16( sum_j (dg W_gate[e]^T + du W_up[e]^T) ), j ascending
 *   dW_gate[e] = bf16( sum_r X[t]^T dg ),  dW_up[e] = bf16( sum_r X[t]^T du )
 *   dW_down[e] = bf16( sum_r h^T dO )      (all sums in fp32, fixed order;
 *                                           experts without rows get zeros)
 *   X, dY [T, H] bf16;  topk_w [T, k] fp32;  dispatch arrays as above
 *   Wg_t, Wu_t [E, I, H], Wd_t [E, H, I] bf16: the packed weights moe_expert_mlp takes
 *            (moe_pack_weights of W_gate, W_up [E, H, I] and W_down [E, I, H]); no other
 *            copy of the weights is needed
 *   dX [T, H], dW_gate, dW_up [E, H, I], dW_down [E, I, H] bf16 out;
 *   d_topk_w [T, k] fp32 out
 *   ws, ws_bytes   workspace of moe_workspace_size(MOE_CALL_BACKWARD)
 * MOE_ACT_RELU2 has no gate: du = dh * 2 max(U, 0), dX sums du W_up[e]^T only,
 * Wg_t and dW_gate may be NULL and dW_gate is not written.
 */
MOE_API moe_status moe_backward(const moe_problem* p, const void* X, const void* dY,
                                const float* topk_w, const int32_t* row_token,
                                const int32_t* row_slot, const int32_t* slot_row,
                                const int32_t* expert_offsets, const void* Wg_t,
                                const void* Wu_t, const void* Wd_t, void* dX, void* dW_gate,
                                void* dW_up, void* dW_down, float* d_topk_w, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * Training forward that keeps its projections for the backward.  The pages'
 * backward recomputes G and U (LigerCute "Backward pass": activation
 * recomputation) to save memory; a GPU with 288 GB of HBM holds a step's fp32
 * G and U (T*k*2I*4 bytes: 512 MiB for 8,192 tokens, top-8, I = 1024) at no
 * cost worth the recompute GEMM, so this pair of calls trades that memory for
 * the 4*T*k*H*I FLOP of the recompute.
 * moe_expert_mlp_save: moe_expert_mlp (bf16 only, the row-grouped GEMMs for
 * every T, no workspace) that also writes
 *   GU_rows  [T*k, 2I] fp32 out: G = X[row_token[r]] W_gate[e] in columns [0, I)
 *            and U = X[row_token[r]] W_up[e] in columns [I, 2I) of every routed
 *            row r, the fp32 accumulations from which h is formed (MOE_ACT_RELU2:
 *            U only; columns [0, I) are not written)
 * Other arguments, results and errors as moe_expert_mlp (bf16, Sg = Su = Sd = NULL);
 * MXFP8 problems give MOE_ERR_UNSUPPORTED_SHAPE.
 */
MOE_API moe_status moe_expert_mlp_save(const moe_problem* p, const void* X, const int32_t* row_token,
                                       const int32_t* expert_offsets, const void* Wg_t,
                                       const void* Wu_t, const void* Wd_t, void* H_rows,
                                       void* O_rows, float* GU_rows, void* stream);

/*
 * moe_backward with G and U read from GU_rows (as moe_expert_mlp_save wrote it
 * for the same problem, dispatch and weights) instead of recomputed.  The
 * results are those of moe_backward: dX and the weight gradients from the same
 * operands, d_topk_w[s] = <h, P> summed per row in a fixed order of its own.
 *   GU_rows  [T*k, 2I] fp32 in
 * Other arguments, workspace (moe_workspace_size(MOE_CALL_BACKWARD)) and errors
 * as moe_backward.
 */
MOE_API moe_status moe_backward_saved(const moe_problem* p, const void* X, const void* dY,
                                      const float* topk_w, const int32_t* row_token,
                                      const int32_t* row_slot, const int32_t* slot_row,
                                      const int32_t* expert_offsets, const void* Wg_t,
                                      const void* Wu_t, const void* Wd_t, const float* GU_rows,
                                      void* dX, void* dW_gate, void* dW_up, void* dW_down,
                                      float* d_topk_w, void* ws, size_t ws_bytes, void* stream);

/*
 * Standalone grouped GEMM (LightMoE "Grouped GEMM": contiguous expert-major
 * rows, m_indptr of E+1 int32 offsets, zero-row experts valid, b as
 * [num_experts, N, K]; the same kernels as the expert MLP's down projection):
 *   C[r] = bf16( A[r] B_t[e]^T )   for m_indptr[e] <= r < m_indptr[e+1]
 * with fp32 accumulation.
 *   dtype        MOE_DTYPE_BF16 or MOE_DTYPE_MXFP8
 *   m_indptr     [E+1] int32 (device): m_indptr[0] = 0, non-decreasing,
 *                m_indptr[E] <= M; rows past m_indptr[E] are not written
 *   bf16:  A [M, K] bf16, B_t [E, N, K] bf16 (moe_pack_weights of [E, K, N]);
 *          SA, SB must be NULL
 *   MXFP8: A [M, K] and B_t [E, N, K] E4M3 codes with SA [M, K/32] and
 *          SB [E, N, K/32] E8M0 scales (moe_mx_quantize)
 *   C      [M, N] bf16 out
 *   Limits: 1 <= E <= 1024; 0 <= M < 2^31 with M*K < 2^31; N and K multiples
 *   of 64 (MXFP8: 128).  M = 0 is valid and does nothing.
 */
MOE_API moe_status moe_grouped_gemm(int32_t dtype, const int32_t* m_indptr, int32_t E, int64_t M,
                                    int32_t N, int32_t K, const void* A, const uint8_t* SA,
                                    const void* B_t, const uint8_t* SB, void* C, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
