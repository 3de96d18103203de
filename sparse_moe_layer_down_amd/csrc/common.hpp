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

#define LMOE_DEV __device__ __forceinline__

template <typename T> LMOE_DEV T from_f32(float v);
template <> LMOE_DEV float from_f32<float>(float v) { return v; }
template <> LMOE_DEV bf16 from_f32<bf16>(float v) { return (bf16)v; }  // round to nearest even

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

// Work-group -> logical tile mapping aware of the 8 XCDs: consecutive work-group
// ids are dispatched round-robin over the XCDs, so chunks of `chunk` consecutive
// logical tiles are handed to one XCD (shared operands then meet in that XCD's
// L2), and the chunks themselves rotate over the XCDs.  The grid must be a
// multiple of 8 * chunk.
LMOE_DEV int xcd_logical_tile(int pid, int chunk) {
  const int x = pid & 7, i = pid >> 3;
  const int q = (i / chunk) * 8 + x;
  return q * chunk + (i % chunk);
}

LMOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace lmoe
