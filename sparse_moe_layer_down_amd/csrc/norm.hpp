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
  const int nrows = k + n_shared;
  float u[CPT][8];
#pragma unroll
  for (int q = 0; q < CPT; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) u[q][i] = 0.0f;
  // rows four at a time so their loads are in flight together: the k routed
  // rows of t (through slot_row), then its shared-expert rows
  for (int r0 = 0; r0 < nrows; r0 += 4) {
    int64_t row[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = min(r0 + j, nrows - 1);
      row[j] = r < k ? (int64_t)slot_row[t * k + r] : (int64_t)T_ * k + (int64_t)(r - k) * T_ + t;
    }
    float y[4][CPT][8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int ch = min((int)threadIdx.x + q * 256, nch - 1);
        load8_f32(ystage + row[j] * L + ch * 8, y[j][q]);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (r0 + j >= nrows) break;
#pragma unroll
      for (int q = 0; q < CPT; ++q)
#pragma unroll
        for (int i = 0; i < 8; ++i) u[q][i] += y[j][q][i];
    }
  }
  float ss = 0.0f;
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    if ((int)threadIdx.x + q * 256 < nch) {
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
