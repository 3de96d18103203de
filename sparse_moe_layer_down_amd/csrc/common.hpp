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
LMOE_DEV float sigmoidf_(float x) { return 1.0f / (1.0f + expf(-x)); }
LMOE_DEV float softcapf_(float x, float beta) { return beta * tanhf(x / beta); }
LMOE_DEV float situf_(float x, float beta) { return softcapf_(x, beta) * sigmoidf_(x); }

LMOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace lmoe
