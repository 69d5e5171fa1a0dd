// Internal helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 pair -> packed bf16 pair (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// fp32 -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// Four fp32 values -> four bf16 at dst (8-byte aligned).
__device__ __forceinline__ void store_bf16x4(uint16_t* dst, float a, float b, float c, float d) {
  uint2 v;
  v.x = pack_bf16x2(a, b);
  v.y = pack_bf16x2(c, d);
  *reinterpret_cast<uint2*>(dst) = v;
}

// sigmoid / silu in fp32 with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float sigmoid_f32(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_f32(float x) { return x * sigmoid_f32(x); }

// Activations h = f(g, u) (the moe_activation codes) and their partial
// derivatives, in fp32.  Clamps pass the gradient where their argument lies
// inside the bounds, the bounds included.  ReLU^2 is ungated (h = f(u)): its
// kernels have no gate operand and call relu2 / relu2_grad.
enum : int { ACT_SWIGLU = 0, ACT_SWIGLU_CLAMP = 1, ACT_SWIGLU_OAI = 2, ACT_GEGLU = 3, ACT_REGLU = 4, ACT_RELU2 = 5 };
__host__ __device__ constexpr bool act_gated(int act) { return act != ACT_RELU2; }
__device__ __forceinline__ float relu2(float u) {
  const float r = fmaxf(u, 0.f);
  return r * r;
}
__device__ __forceinline__ float relu2_grad(float u) { return 2.f * fmaxf(u, 0.f); }
// Kernels take the activation as a template constant ACTK: ACT_SWIGLU for the
// default path (nothing else compiled in), ACT_ANY to switch on the run-time code.
constexpr int ACT_ANY = -1;
__device__ __forceinline__ int act_code(int actk, int runtime) { return actk == ACT_ANY ? runtime : actk; }
constexpr float OAI_ALPHA = 1.702f;
constexpr float INV_SQRT2 = 0.70710678118654752f;
constexpr float INV_SQRT_2PI = 0.39894228040143268f;

__device__ __forceinline__ float gated_act(float g, float u, int act, float lim) {
  switch (act) {
    case ACT_SWIGLU_CLAMP: return silu_f32(fminf(g, lim)) * fminf(fmaxf(u, -lim), lim);
    case ACT_SWIGLU_OAI: {
      const float gc = fminf(g, lim);
      return gc * sigmoid_f32(OAI_ALPHA * gc) * (fminf(fmaxf(u, -lim), lim) + 1.f);
    }
    case ACT_GEGLU: return 0.5f * g * (1.f + erff(g * INV_SQRT2)) * u;
    case ACT_REGLU: return fmaxf(g, 0.f) * u;
    default: return silu_f32(g) * u;
  }
}

// h = f(g, u), fg = df/dg, fu = df/du.
__device__ __forceinline__ void gated_act_grad(float g, float u, int act, float lim, float& h, float& fg,
                                               float& fu) {
  switch (act) {
    case ACT_SWIGLU_CLAMP:
    case ACT_SWIGLU_OAI: {
      const float gc = fminf(g, lim), uc = fminf(fmaxf(u, -lim), lim);
      const float pg = g <= lim ? 1.f : 0.f, pu = (u >= -lim && u <= lim) ? 1.f : 0.f;
      if (act == ACT_SWIGLU_CLAMP) {
        const float s = sigmoid_f32(gc);
        h = gc * s * uc;
        fg = uc * (s * (1.f + gc * (1.f - s))) * pg;
        fu = gc * s * pu;
      } else {
        const float s = sigmoid_f32(OAI_ALPHA * gc);
        h = gc * s * (uc + 1.f);
        fg = (s + OAI_ALPHA * gc * s * (1.f - s)) * (uc + 1.f) * pg;
        fu = gc * s * pu;
      }
      return;
    }
    case ACT_GEGLU: {
      const float Phi = 0.5f * (1.f + erff(g * INV_SQRT2));
      h = g * Phi * u;
      fg = (Phi + g * INV_SQRT_2PI * __expf(-0.5f * g * g)) * u;
      fu = g * Phi;
      return;
    }
    case ACT_REGLU:
      h = fmaxf(g, 0.f) * u;
      fg = g > 0.f ? u : 0.f;
      fu = fmaxf(g, 0.f);
      return;
    default: {
      const float s = sigmoid_f32(g);
      h = g * s * u;
      fg = u * (s * (1.f + g * (1.f - s)));
      fu = g * s;
    }
  }
}

// fg = df/dg alone, computed as gated_act_grad computes it (the same value, bit for bit).
__device__ __forceinline__ float gated_act_dg(float g, float u, int act, float lim) {
  switch (act) {
    case ACT_SWIGLU_CLAMP:
    case ACT_SWIGLU_OAI: {
      const float gc = fminf(g, lim), uc = fminf(fmaxf(u, -lim), lim);
      const float pg = g <= lim ? 1.f : 0.f;
      if (act == ACT_SWIGLU_CLAMP) {
        const float s = sigmoid_f32(gc);
        return uc * (s * (1.f + gc * (1.f - s))) * pg;
      }
      const float s = sigmoid_f32(OAI_ALPHA * gc);
      return (s + OAI_ALPHA * gc * s * (1.f - s)) * (uc + 1.f) * pg;
    }
    case ACT_GEGLU: {
      const float Phi = 0.5f * (1.f + erff(g * INV_SQRT2));
      return (Phi + g * INV_SQRT_2PI * __expf(-0.5f * g * g)) * u;
    }
    case ACT_REGLU: return g > 0.f ? u : 0.f;
    default: {
      const float s = sigmoid_f32(g);
      return u * (s * (1.f + g * (1.f - s)));
    }
  }
}

// fu = df/du alone, computed as gated_act_grad computes it (the same value, bit for bit).
__device__ __forceinline__ float gated_act_du(float g, float u, int act, float lim) {
  switch (act) {
    case ACT_SWIGLU_CLAMP:
    case ACT_SWIGLU_OAI: {
      const float gc = fminf(g, lim);
      const float pu = (u >= -lim && u <= lim) ? 1.f : 0.f;
      const float s = act == ACT_SWIGLU_CLAMP ? sigmoid_f32(gc) : sigmoid_f32(OAI_ALPHA * gc);
      return gc * s * pu;
    }
    case ACT_GEGLU: {
      const float Phi = 0.5f * (1.f + erff(g * INV_SQRT2));
      return g * Phi;
    }
    case ACT_REGLU: return fmaxf(g, 0.f);
    default: return g * sigmoid_f32(g);
  }
}

}  // namespace moe
