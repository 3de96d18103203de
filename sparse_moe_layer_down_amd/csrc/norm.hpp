// Combine + RMSNorm: the aggregated latent of token t is the sum, in fp32, of
// its k routed rows (staged by the W3 epilogue already scaled by their routing
// weights) and its n_shared shared-expert rows (rows T*k + s*T + t), all staged
// in fp16 for bf16 inputs and fp32 for fp32 inputs.  The single
// retained RMSNorm then gives v = gain * u / sqrt(mean(u^2) + eps)
// ("Kimi K3 Architecture Deep Dive" §2: one RMS norm before the
// up-projection; LeiPhone report "Keeping the numbers in range": after
// aggregation, before projecting back up); with no_norm set (the ablation of
// that norm) v = u.  u stays in registers between the
// two passes.  Up to L = 4096 one wave handles one token (CPT 16-byte chunks
// of the row per lane, no block barrier); wider rows use one work-group per
// token.
#pragma once
#include "common.hpp"

namespace lmoe {

// 8 staged elements -> fp32 with a non-temporal load: every staged row is read
// exactly once, so it should not displace cached data
LMOE_DEV void load8_f32_stream(const f16 *p, float *o) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
  const f16x8 b = __builtin_bit_cast(f16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)b[i];
}
LMOE_DEV void load8_f32_stream(const bf16 *p, float *o) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
  const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (float)b[i];
}
LMOE_DEV void load8_f32_stream(const float *p, float *o) {
  const f32x4 a = __builtin_nontemporal_load((const f32x4 *)p), b = __builtin_nontemporal_load((const f32x4 *)(p + 4));
#pragma unroll
  for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
}

// One wave per token (four tokens per 256-thread work-group); lane l owns the
// chunks l, l + 64, ..., and two rows' loads are in flight together.
template <typename T, typename TS, int CPT>
__global__ __launch_bounds__(256) void combine_rmsnorm_wave_kernel(const TS *__restrict__ ystage,
                                                                   const int32_t *__restrict__ slot_row,
                                                                   const T *__restrict__ gain, T *__restrict__ v,
                                                                   int T_, int L, int k, int n_shared, float eps,
                                                                   int no_norm) {
  constexpr int RIF = 2;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;  // the whole wave: no barrier follows
  const int lane = threadIdx.x & 63;
  const int nch = L / 8;
  const int nrows = k + n_shared;
  float u[CPT][8];
#pragma unroll
  for (int q = 0; q < CPT; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) u[q][i] = 0.0f;
  // the k routed row indices of t, one per lane (k <= 64), read up front
  const int my_row = lane < k ? slot_row[t * k + lane] : 0;
  for (int r0 = 0; r0 < nrows; r0 += RIF) {
    int64_t row[RIF];
#pragma unroll
    for (int j = 0; j < RIF; ++j) {
      const int r = min(r0 + j, nrows - 1);
      row[j] = r < k ? (int64_t)__builtin_amdgcn_readlane(my_row, r) : (int64_t)T_ * k + (int64_t)(r - k) * T_ + t;
    }
    float y[RIF][CPT][8];
#pragma unroll
    for (int j = 0; j < RIF; ++j)
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int ch = min(lane + q * 64, nch - 1);
        load8_f32_stream(ystage + row[j] * L + ch * 8, y[j][q]);
      }
#pragma unroll
    for (int j = 0; j < RIF; ++j) {
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
    if (lane + q * 64 < nch) {
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += u[q][i] * u[q][i];
    }
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / sqrtf(ss / (float)L + eps);
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int ch = lane + q * 64;
    if (ch < nch) {
      if (no_norm) {  // the ablation: v = u
        store8(v + t * L + ch * 8, u[q]);
        continue;
      }
      float g[8], o[8];
      load8_f32(gain + ch * 8, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = g[i] * (u[q][i] * rstd);
      store8(v + t * L + ch * 8, o);
    }
  }
}

template <typename T, typename TS, int CPT>
__global__ __launch_bounds__(256) void combine_rmsnorm_kernel(const TS *__restrict__ ystage,
                                                              const int32_t *__restrict__ slot_row,
                                                              const T *__restrict__ gain, T *__restrict__ v,
                                                              int T_, int L, int k, int n_shared, float eps,
                                                              int no_norm) {
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
      if (no_norm) {  // the ablation: v = u
        store8(v + t * L + ch * 8, u[q]);
        continue;
      }
      float g[8], o[8];
      load8_f32(gain + ch * 8, g);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = g[i] * (u[q][i] * rstd);
      store8(v + t * L + ch * 8, o);
    }
  }
}

// In-place row RMSNorm with unit gain, z[t] <- z[t] / sqrt(mean(z[t]^2) + eps):
// the extra norm after the down-projection that the layer leaves out ("Kimi K3
// Architecture Deep Dive" §2 keeps only the norm before the up-projection), for
// its ablation.  One wave per row, four rows per work-group, rows strided over
// the grid; each lane reads its 8-element chunks twice (the second read hits
// the caches), since this runs only in the ablation.  L is a multiple of 8.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_rows_kernel(T *__restrict__ z, int T_, int L, float eps) {
  const int lane = threadIdx.x & 63;
  const int nch = L / 8;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T_; t += (int64_t)gridDim.x * 4) {
    T *row = z + t * L;
    float ss = 0.0f;
    for (int ch = lane; ch < nch; ch += 64) {
      float a[8];
      load8_f32(row + ch * 8, a);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += a[i] * a[i];
    }
    ss = wave_sum(ss);
    const float rstd = 1.0f / sqrtf(ss / (float)L + eps);
    for (int ch = lane; ch < nch; ch += 64) {
      float a[8];
      load8_f32(row + ch * 8, a);
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] *= rstd;
      store8(row + ch * 8, a);
    }
  }
}

}  // namespace lmoe
