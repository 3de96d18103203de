// Shared device helpers for the LatentMoE kernels (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lmoe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

#define LMOE_DEV __device__ __forceinline__

template <typename T> LMOE_DEV T from_f32(float v);
template <> LMOE_DEV float from_f32<float>(float v) { return v; }
template <> LMOE_DEV bf16 from_f32<bf16>(float v) { return (bf16)v; }  // round to nearest even
template <> LMOE_DEV f16 from_f32<f16>(float v) { return (f16)v; }     // RNE; beyond +-65504 -> +-inf

template <typename T> LMOE_DEV float to_f32(T v) { return (float)v; }

// 8 consecutive work-dtype elements (16 B for bf16, 32 B for fp32) -> fp32
LMOE_DEV void load8_f32(const bf16 *p, float *o) {
  u32x4 v = *(const u32x4 *)p;
  bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)b[i];
}
LMOE_DEV void load8_f32(const float *p, float *o) {
  const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
}
LMOE_DEV void load8_f32(const f16 *p, float *o) {
  u32x4 v = *(const u32x4 *)p;
  f16x8 b = __builtin_bit_cast(f16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)b[i];
}
// 4 consecutive elements from fp32 values (one 16-B or 8-B store)
LMOE_DEV void store4(float *p, const float *v) { *(f32x4 *)p = f32x4{v[0], v[1], v[2], v[3]}; }
LMOE_DEV void store4(bf16 *p, const float *v) {
  const bf16x4 b = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *(u32x2 *)p = __builtin_bit_cast(u32x2, b);
}
LMOE_DEV void store4(f16 *p, const float *v) {
  const f16x4 b = {(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
  *(u32x2 *)p = __builtin_bit_cast(u32x2, b);
}
LMOE_DEV void store8(bf16 *p, const float *v) {
  bf16x8 b;
#pragma unroll
  for (int i = 0; i < 8; ++i) b[i] = (bf16)v[i];
  *(u32x4 *)p = __builtin_bit_cast(u32x4, b);
}
LMOE_DEV void store8(float *p, const float *v) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  *(f32x4 *)p = a;
  *(f32x4 *)(p + 4) = b;
}

// softcap(x; beta) = beta * tanh(x / beta); SiTU(x; beta) = softcap(x; beta) * sigmoid(x)
// ("Kimi K3 Architecture Deep Dive" §1)
// The router's sigmoid uses the library expf (its scores feed the top-k and
// the QB histogram); the gate epilogue, evaluated for every hidden unit of
// every dispatched row, uses the hardware exp2 / reciprocal.  With y = x / beta:
//   softcap = beta sign(y) (1 - e^{-2|y|}) / (1 + e^{-2|y|})          for |y| >= 3/8,
//   softcap = x (1 - y^2/3 + 2y^4/15 - 17y^6/315 + 62y^8/2835 - 1382y^10/155925)  below
// (tanh's odd Taylor series divided by y; the truncation error there is under
// 2e-8 relative), so the first form never cancels by more than a factor of
// 3.5; both stay within about 3e-7 relative of beta tanh(x / beta), NaN and
// +-inf included (but beta = +inf turns an infinite x into NaN: y = inf * 0).
// beta = +inf gives y = 0 for finite x and so exactly x, the uncapped
// limit: SiTU becomes SiLU and SiTU-GLU becomes SwiGLU, the gate the caps are
// measured against.
LMOE_DEV float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
LMOE_DEV float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
LMOE_DEV float sigmoid_hw(float x) { return __builtin_amdgcn_rcpf(1.0f + exp_hw(-x)); }
LMOE_DEV float softcapf_(float x, float beta) {
  const float y = x * (1.0f / beta);  // 1/beta is hoisted
  const float a = fabsf(y);
  const float t = exp_hw(-2.0f * a);
  const float big = (1.0f - t) * __builtin_amdgcn_rcpf(1.0f + t);
  const float y2 = y * y;
  float q = -1382.0f / 155925.0f;
  q = 62.0f / 2835.0f + y2 * q;
  q = -17.0f / 315.0f + y2 * q;
  q = 2.0f / 15.0f + y2 * q;
  q = -1.0f / 3.0f + y2 * q;
  q = 1.0f + y2 * q;
  return a < 0.375f ? x * q : beta * copysignf(big, y);
}
LMOE_DEV float situf_(float x, float beta) { return softcapf_(x, beta) * sigmoid_hw(x); }

LMOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace lmoe
