// Combine + RMSNorm: the aggregated latent of token t is the sum, in fp32, of
// its k routed rows (staged by the W3 epilogue already scaled by their routing
// weights) and its n_shared shared-expert rows (rows T*k + s*T + t), all staged
// in fp16 for bf16 inputs and fp32 for fp32 inputs.  The single
// retained RMSNorm then gives v = gain * u / sqrt(mean(u^2) + eps)
// ("Kimi K3 Architecture Deep Dive" §2: one RMS norm before the
// up-projection; LeiPhone report "Keeping the numbers in range": after
// aggregation, before projecting back up).  One work-group per token; u stays
// in registers between the two passes.
#pragma once
#include "common.hpp"

namespace lmoe {

template <typename T, typename TS, int CPT>
__global__ __launch_bounds__(256) void combine_rmsnorm_kernel(const TS *__restrict__ ystage,
                                                              const int32_t *__restrict__ slot_row,
                                                              const T *__restrict__ gain, T *__restrict__ v,
                                                              int T_, int L, int k, int n_shared, float eps) {
  __shared__ float red[4];
  const int64_t t = blockIdx.x;
  const int nch = L / 8;
  float u[CPT][8];
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int ch = threadIdx.x + q * 256;
#pragma unroll
    for (int i = 0; i < 8; ++i) u[q][i] = 0.0f;
    if (ch < nch) {
      for (int sh = 0; sh < n_shared; ++sh) {
        const int64_t row = (int64_t)T_ * k + (int64_t)sh * T_ + t;
        float y[8];
        load8_f32(ystage + row * L + ch * 8, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[q][i] += y[i];
      }
      for (int r = 0; r < k; ++r) {
        const int64_t row = slot_row[t * k + r];
        float y[8];
        load8_f32(ystage + row * L + ch * 8, y);
#pragma unroll
        for (int i = 0; i < 8; ++i) u[q][i] += y[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += u[q][i] * u[q][i];
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = red[0] + red[1] + red[2] + red[3];
  const float rstd = 1.0f / sqrtf(tot / (float)L + eps);
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int ch = threadIdx.x + q * 256;
    if (ch < nch) {
      float g[8], o[8];
      load8_f32(gain + ch * 8, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = g[i] * (u[q][i] * rstd);
      store8(v + t * L + ch * 8, o);
    }
  }
}

}  // namespace lmoe
