// Backward-pass kernels of the Stable LatentMoE layer (the matrix products run
// in the MFMA GEMM of gemm.hpp; these kernels prepare its operands and do the
// element-wise and per-token steps).
//
//   transpose_kernel   out[c][kk] = scale(row) * in[row(kk)][c], 64-row tiles of
//                      up to 256 columns through LDS with 16-byte global accesses: plain
//                      transposes (row(kk) = kk, zero past R) and, for the
//                      experts' weight gradients, gathered ones whose 64-wide
//                      column blocks each belong to one expert's segment of rows
//   bwd_scan_kernel    per-expert segments of the padded row axis of those
//                      gathered operands (whole 64-row blocks, at least two per
//                      expert), the K-range tile table and the column-block table
//   norm_bwd_wave_kernel  one wavefront per token: the aggregated latent u is
//                      summed again from the forward's staged rows, then the
//                      RMSNorm backward ("Kimi K3 Architecture Deep Dive" §2)
//                        du = (gamma dv - u_hat mean(gamma dv u_hat)) / r,
//                      dv * u_hat for the gain's gradient, and the routing
//                      weights' gradients dg_j = du . o_j (o_j = staged row / g_j)
//   colsum_*_kernel    gain gradient: column sums of dv * u_hat over tokens
//                      (row slices, then the slices' sums, both in fixed order)
//   router_bwd_kernel  one wavefront per token: g_j = s_j / S over the chosen
//                      experts, so ds_j = (dg_j - sum_j' dg_j' g_j') / S and
//                      dl_j = ds_j s_j (1 - s_j); the row of dl is written dense
//                      (zeros off the chosen experts: selection has no gradient)
#pragma once
#include "common.hpp"

namespace lmoe {

constexpr int TP_TILE = 64;

// Tiles of 64 rows (blockIdx.y: 64 output columns kk) by CT x 64 columns c of
// the input (blockIdx.x), blockIdx.z: batch.  Without a block table, output
// column kk takes input row kk (zero for kk >= R).  With one (int4 per 64-column
// block: {first input row, valid rows, -, -}), column kk = 64 b + q takes input
// row rows[first + q] (or first + q without a row map) for q < valid and zero
// beyond; blocks at or past *nblocks are skipped; rscale[first + q] scales the
// row.  C, ld_in and ld_out are multiples of the 16-byte element count; out
// columns are written in whole 64-wide blocks (ld_out >= the padded column
// count).  A thread issues all its loads of the CT tiles (the same rows, CT
// column pieces each) before its LDS stores, so a block waits for memory once;
// 256 threads.
template <typename T, int CT>
__global__ __launch_bounds__(256) void transpose_kernel(const T *__restrict__ in, int64_t ld_in, int64_t in_bs,
                                                        T *__restrict__ out, int64_t ld_out, int64_t out_bs, int R,
                                                        int C, const int4 *__restrict__ blocks,
                                                        const int32_t *__restrict__ nblocks,
                                                        const int32_t *__restrict__ rows,
                                                        const float *__restrict__ rscale) {
  constexpr int EPT = 16 / (int)sizeof(T);       // elements per 16 bytes
  constexpr int CPR = TP_TILE / EPT;              // 16-byte chunks per tile row
  constexpr int PER = TP_TILE * CPR / 256;        // a thread's chunks of one tile
  __shared__ __attribute__((aligned(16))) T tile[CT][TP_TILE][TP_TILE + EPT];
  const int c0 = blockIdx.x * TP_TILE * CT;
  const int kb = blockIdx.y;
  if (blocks && kb >= *nblocks) return;  // uniform over the work-group
  const int64_t b = blockIdx.z;
  in += b * in_bs;
  out += b * out_bs;
  int first = kb * TP_TILE, valid = min(TP_TILE, R - kb * TP_TILE);
  if (blocks) {
    const int4 e = blocks[kb];
    first = e.x;
    valid = e.y;
  }
  // the thread's rows (the same in every column tile): chunk i = tid + 256 p is
  // row q = i / CPR, 16-byte chunk i % CPR of the tile's 64 columns
  int src[PER];
  float sc[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) {
    const int q = ((int)threadIdx.x + 256 * p) / CPR;
    src[p] = q < valid ? (blocks && rows ? rows[first + q] : first + q) : -1;
    sc[p] = rscale && q < valid ? rscale[first + q] : 1.0f;
  }
  u32x4 v[CT][PER];
#pragma unroll
  for (int t = 0; t < CT; ++t)
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int c = c0 + t * TP_TILE + (((int)threadIdx.x + 256 * p) % CPR) * EPT;
      v[t][p] = u32x4{0u, 0u, 0u, 0u};
      if (src[p] >= 0 && c < C) v[t][p] = *(const u32x4 *)(in + (int64_t)src[p] * ld_in + c);
    }
#pragma unroll
  for (int t = 0; t < CT; ++t)
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = (int)threadIdx.x + 256 * p;
      u32x4 w = v[t][p];
      if (rscale) {
        T *e = (T *)&w;
#pragma unroll
        for (int j = 0; j < EPT; ++j) e[j] = from_f32<T>(to_f32(e[j]) * sc[p]);
      }
      *(u32x4 *)&tile[t][i / CPR][(i % CPR) * EPT] = w;
    }
  __syncthreads();
  // store: output row c (64 per tile) x CPR chunks of consecutive kk
#pragma unroll
  for (int t = 0; t < CT; ++t)
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = (int)threadIdx.x + 256 * p;
      const int cc = i / CPR, ch = i % CPR;
      const int c = c0 + t * TP_TILE + cc;
      if (c >= C) continue;
      u32x4 w;
      T *e = (T *)&w;
#pragma unroll
      for (int j = 0; j < EPT; ++j) e[j] = tile[t][ch * EPT + j][cc];
      *(u32x4 *)(out + (int64_t)c * ld_out + (int64_t)kb * TP_TILE + ch * EPT) = w;
    }
}

// Segments of the experts' padded row axis (one work-group of 1024 threads).
// Segment e < n is routed expert e (its counts[e] dispatched rows, starting at
// offs[e]); segment n + s is shared expert s (T rows starting at T k + s T).
// Each segment is padded to whole 64-row blocks.  Outputs: entries[e] =
// {e, first K step, K steps, 0} (steps of `bke` elements) for every segment,
// empty ones included (their weight gradient is then a tile of zeros);
// blocks[b] = {first expert row, valid rows, e, 0} for every 64-row block;
// nblocks[0] = the block count, nblocks[1] = the entry count; sched[0 .. nsched)
// zeroed (tile counters).
__global__ __launch_bounds__(1024) void bwd_scan_kernel(const int32_t *__restrict__ counts,
                                                        const int32_t *__restrict__ offs, int n, int n_shared, int T,
                                                        int k, int bke, int4 *__restrict__ entries,
                                                        int4 *__restrict__ blocks, int32_t *__restrict__ nblocks,
                                                        int32_t *__restrict__ sched, int nsched) {
  __shared__ int32_t sc[1024];
  const int nseg = n + n_shared;
  const int per = (nseg + 1023) / 1024;  // segments per thread (<= 2)
  int mine[2] = {0, 0};
  int tot = 0;
  for (int j = 0; j < per; ++j) {
    const int e = threadIdx.x * per + j;
    const int R = e < n ? counts[e] : (e < nseg ? T : 0);
    // at least two blocks per segment (zero blocks past its rows), so that every
    // K-range tile has at least two K steps and the GEMM can prefetch across tiles
    mine[j] = e < nseg ? max(2, (R + TP_TILE - 1) / TP_TILE) : 0;
    tot += mine[j];
  }
  sc[threadIdx.x] = tot;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = threadIdx.x >= o ? sc[threadIdx.x - o] : 0;
    __syncthreads();
    sc[threadIdx.x] += a;
    __syncthreads();
  }
  int base = sc[threadIdx.x] - tot;  // first block of this thread's first segment
  const int spb = TP_TILE / bke;     // GEMM K steps per 64-row block
  for (int j = 0; j < per; ++j) {
    const int e = threadIdx.x * per + j;
    if (e >= nseg) break;
    const int R = e < n ? counts[e] : T;
    const int row0 = e < n ? offs[e] : T * k + (e - n) * T;
    entries[e] = make_int4(e, base * spb, mine[j] * spb, 0);
    for (int q = 0; q < mine[j]; ++q)
      blocks[base + q] = make_int4(row0 + q * TP_TILE, max(0, min(TP_TILE, R - q * TP_TILE)), e, 0);
    base += mine[j];
  }
  if (threadIdx.x == 1023) {
    nblocks[0] = sc[1023];
    nblocks[1] = nseg;
  }
  for (int i = threadIdx.x; i < nsched; i += blockDim.x) sched[i] = 0;
}

// RMSNorm backward of one token per wavefront (lane l owns the 8-element
// chunks l, l + 64, ...; L <= 4096).  u is re-summed from the staged rows in
// the forward's order.  Writes du (fp32, and in the work dtype for the matrix
// products), dv * u_hat (fp32, for the gain's gradient) and dg[t][j] for the k
// routed slots.  no_norm: the layer had no norm (v = u), so du = dv.
template <typename T, typename TS, int CPT>
__global__ __launch_bounds__(256) void norm_bwd_wave_kernel(const TS *__restrict__ ystage,
                                                            const int32_t *__restrict__ slot_row,
                                                            const float *__restrict__ gw, const T *__restrict__ gain,
                                                            const float *__restrict__ dv, float *__restrict__ du32,
                                                            T *__restrict__ du, float *__restrict__ prod,
                                                            float *__restrict__ dg, int T_, int L, int k,
                                                            int n_shared, float eps, int no_norm) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;  // the whole wave: no barrier follows
  const int lane = threadIdx.x & 63;
  const int nch = L / 8;
  const int nrows = k + n_shared;
  const int my_row = lane < k ? slot_row[t * k + lane] : 0;
  auto row_of = [&](int r) -> int64_t {
    return r < k ? (int64_t)__builtin_amdgcn_readlane(my_row, r) : (int64_t)T_ * k + (int64_t)(r - k) * T_ + t;
  };
  float u[CPT][8], h[CPT][8];
#pragma unroll
  for (int q = 0; q < CPT; ++q)
#pragma unroll
    for (int i = 0; i < 8; ++i) u[q][i] = 0.0f;
  // u: the token's staged rows summed in fp32, in the forward's order, two
  // rows' loads in flight together
  for (int r0 = 0; r0 < nrows; r0 += 2) {
    const int64_t row0 = row_of(r0), row1 = row_of(min(r0 + 1, nrows - 1));
    float y[2][CPT][8];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int ch = min(lane + q * 64, nch - 1);
      load8_f32(ystage + row0 * L + ch * 8, y[0][q]);
      load8_f32(ystage + row1 * L + ch * 8, y[1][q]);
    }
    const bool two = r0 + 1 < nrows;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u[q][i] += y[0][q][i];
        if (two) u[q][i] += y[1][q][i];
      }
  }
  // dv -> h
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int ch = min(lane + q * 64, nch - 1);
    load8_f32(dv + t * L + ch * 8, h[q]);
  }
  if (!no_norm) {
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      if (lane + q * 64 < nch) {
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += u[q][i] * u[q][i];
      }
    ss = wave_sum(ss);
    const float rinv = 1.0f / sqrtf(ss / (float)L + eps);
    // u_hat = u / r; h = gain * dv; c = mean(h * u_hat); prod = dv * u_hat
    float c = 0.0f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int ch = lane + q * 64;
      if (ch >= nch) continue;
      float gm[8], pr[8];
      load8_f32(gain + ch * 8, gm);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        u[q][i] *= rinv;
        pr[i] = h[q][i] * u[q][i];
        h[q][i] *= gm[i];
        c += h[q][i] * u[q][i];
      }
      store8(prod + t * L + ch * 8, pr);
    }
    c = wave_sum(c) / (float)L;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
#pragma unroll
      for (int i = 0; i < 8; ++i) h[q][i] = (h[q][i] - u[q][i] * c) * rinv;
  }
  // h = du: store it (fp32 and work dtype)
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int ch = lane + q * 64;
    if (ch >= nch) continue;
    store8(du32 + t * L + ch * 8, h[q]);
    store8(du + t * L + ch * 8, h[q]);
  }
  // dg_j = du . o_j where the staged row holds g_j o_j; two rows' loads in
  // flight together, each row's dot product in the same order as alone
  for (int r0 = 0; r0 < k; r0 += 2) {
    const int r1 = min(r0 + 1, k - 1);
    const int64_t row0 = row_of(r0), row1 = row_of(r1);
    float y[2][CPT][8];
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int ch = min(lane + q * 64, nch - 1);
      load8_f32(ystage + row0 * L + ch * 8, y[0][q]);
      load8_f32(ystage + row1 * L + ch * 8, y[1][q]);
    }
    float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      if (lane + q * 64 >= nch) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        acc0 += h[q][i] * y[0][q][i];
        acc1 += h[q][i] * y[1][q][i];
      }
    }
    acc0 = wave_sum(acc0);
    acc1 = wave_sum(acc1);
    if (lane == 0) {
      dg[t * k + r0] = acc0 / gw[t * k + r0];
      if (r0 + 1 < k) dg[t * k + r1] = acc1 / gw[t * k + r1];
    }
  }
}

// Column sums out[c] = sum over rows t of in[t][c] in two fixed-order stages
// (deterministic): work-group (column block x, row slice y) sums its slice of
// rows into part[y][c]; then the slices' partial sums are added in order.
constexpr int COLSUM_SLICES = 64;

__global__ __launch_bounds__(256) void colsum_partial_kernel(const float *__restrict__ in, int rows, int cols,
                                                             float *__restrict__ part) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  const int per = (rows + COLSUM_SLICES - 1) / COLSUM_SLICES;
  const int t0 = blockIdx.y * per, t1 = min(rows, t0 + per);
  float s = 0.0f;
  for (int t = t0; t < t1; ++t) s += in[(int64_t)t * cols + c];
  part[(int64_t)blockIdx.y * cols + c] = s;
}

template <typename T>
__global__ __launch_bounds__(256) void colsum_final_kernel(const float *__restrict__ part, int cols,
                                                           T *__restrict__ out) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= cols) return;
  float s = 0.0f;
  for (int y = 0; y < COLSUM_SLICES; ++y) s += part[(int64_t)y * cols + c];
  out[c] = from_f32<T>(s);
}

template <typename T>
__global__ void fill_zero_kernel(T *__restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = from_f32<T>(0.0f);
}

// Router backward, one wavefront per token (k <= 64): dl[t][0 .. n_pad) in the
// work dtype, dense, zero off the chosen experts.
template <typename T>
__global__ __launch_bounds__(256) void router_bwd_kernel(const float *__restrict__ s, const int32_t *__restrict__ idx,
                                                         const float *__restrict__ gw, const float *__restrict__ dg,
                                                         int T_, int n, int n_pad, int k, T *__restrict__ dl) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_) return;
  const int lane = threadIdx.x & 63;
  int e = -1;
  float sk = 0.0f, g = 0.0f, d = 0.0f;
  if (lane < k) {
    e = idx[t * k + lane];
    sk = s[t * n + e];
    g = gw[t * k + lane];
    d = dg[t * k + lane];
  }
  const float S = wave_sum(sk);
  const float G = wave_sum(d * g);
  const float dl_mine = lane < k ? (d - G) / S * sk * (1.0f - sk) : 0.0f;
  for (int c0 = 0; c0 < n_pad; c0 += 64) {
    const int c = c0 + lane;
    float v = 0.0f;
    for (int j = 0; j < k; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      const float vj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, dl_mine), j));
      v = (ej == c) ? vj : v;
    }
    if (c < n_pad) dl[t * n_pad + c] = from_f32<T>(v);
  }
}

}  // namespace lmoe
