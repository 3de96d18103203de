// Quantile Balancing kernels ("Kimi K3 Architecture Deep Dive" §3: scores in
// [0,1], a fixed B-bin histogram per expert, histograms summed across devices,
// the quantile read from the sum; "Inside K3" section Quantile Balancing;
// LeiPhone report "Keeping the numbers in range": each expert's threshold is
// moved to where it gets its target share).
//
//   qb_hist_kernel   LDS-privatised histogram: a work-group owns EG experts
//                    x a run of tokens, counts in LDS with ds atomics, then adds
//                    its non-zero bins to the global int32 histogram.
//   qb_pool_kernel   pooled histogram sum_e H[e] (int64), one lane per bin.
//   qb_solve_kernel  one wavefront per expert: tail sums G(j) by a wave scan,
//                    j* = max{j : G(j) >= c}, q by linear interpolation inside
//                    bin j*, bias = fp32(tau - q) with tau read the same way
//                    from the pooled histogram.  All counts are integers and
//                    the interpolation is the same sequence of IEEE fp64
//                    operations as the definition, so the result is exact.
#pragma once
#include "common.hpp"

namespace lmoe {

LMOE_DEV int qb_bin(float s, int nbins) {
  const float t = s * (float)nbins;  // one fp32 multiply, round to nearest even
  if (!(t >= 1.0f)) return 0;        // negative, [0,1) and NaN
  if (t >= (float)(nbins - 1)) return nbins - 1;
  return (int)t;                     // t in [1, B-1): truncation is floor
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// grid: (expert groups, token runs); dynamic LDS = eg * nbins * 4 bytes
__global__ __launch_bounds__(256) void qb_hist_kernel(const float *__restrict__ scores, int64_t T, int n,
                                                      int nbins, int eg, int64_t tokens_per_block,
                                                      int32_t *__restrict__ hist) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  int32_t *h = (int32_t *)smem_raw;
  const int e0 = blockIdx.x * eg;
  const int ne = min(eg, n - e0);
  for (int i = threadIdx.x; i < ne * nbins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)blockIdx.y * tokens_per_block;
  const int64_t t1 = min(T, t0 + tokens_per_block);
  const int64_t cnt = (t1 - t0) * ne;
  for (int64_t i = threadIdx.x; i < cnt; i += blockDim.x) {
    const int64_t t = t0 + i / ne;
    const int e = (int)(i % ne);
    atomicAdd(&h[e * nbins + qb_bin(scores[t * n + e0 + e], nbins)], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < ne * nbins; i += blockDim.x) {
    const int v = h[i];
    if (v) atomicAdd(&hist[(int64_t)(e0 + i / nbins) * nbins + (i % nbins)], v);
  }
}

// pooled[j] = sum_e hist[e][j]; block of 256 threads = 64 bins x 4 expert stripes
__global__ __launch_bounds__(256) void qb_pool_kernel(const int32_t *__restrict__ hist, int n, int nbins,
                                                      long long *__restrict__ pooled) {
  __shared__ long long part[4][64];
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  const int stripe = threadIdx.x >> 6;
  long long s = 0;
  if (j < nbins)
    for (int e = stripe; e < n; e += 4) s += hist[(int64_t)e * nbins + j];
  part[stripe][threadIdx.x & 63] = s;
  __syncthreads();
  if (stripe == 0 && j < nbins)
    pooled[j] = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] + part[3][threadIdx.x];
}

// Upper-tail read of one histogram by a full wavefront.  Returns q, or a NaN
// when the histogram is empty.  c = N * k / n where N is the histogram's mass.
template <typename CT>
LMOE_DEV double qb_read_wave(const CT *h, int nbins, long long k, long long n) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int per = (nbins + 63) / 64;
  const int lo = min(lane * per, nbins), hi = min(lo + per, nbins);
  long long mine = 0;
  for (int j = lo; j < hi; ++j) mine += (long long)h[j];
  // suffix sum over lanes above: G at the top of my range
  long long incl = mine;  // inclusive suffix scan (lanes >= me)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long other = __shfl_down(incl, o, 64);
    if (lane + o < 64) incl += other;
  }
  const long long N = __shfl(incl, 0, 64);
  if (N == 0) return __longlong_as_double(0x7FF8000000000000LL);
  const double c = (double)(N * k) / (double)n;
  long long G = incl - mine;  // G(hi)
  int jcand = -1;
  long long Gnext = 0, hj = 0;
  for (int j = hi - 1; j >= lo; --j) {
    const long long gj = G + (long long)h[j];
    if ((double)gj >= c) {
      jcand = j;
      Gnext = G;
      hj = (long long)h[j];
      break;
    }
    G = gj;
  }
  // j* = max over lanes of jcand
  int js = jcand;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) js = max(js, __shfl_xor(js, o, 64));
  // the owning lane holds G(j*+1) and h[j*]; broadcast them
  int owner = (jcand == js) ? lane : 64;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) owner = min(owner, __shfl_xor(owner, o, 64));
  Gnext = __shfl(Gnext, owner, 64);
  hj = __shfl(hj, owner, 64);
  const double frac = (c - (double)Gnext) / (double)hj;
  return ((double)(js + 1) - frac) / (double)nbins;
}

__global__ __launch_bounds__(256) void qb_solve_kernel(const int32_t *__restrict__ hist,
                                                       const long long *__restrict__ pooled, int n, int nbins,
                                                       int k, float *__restrict__ bias) {
#pragma clang fp contract(off)
  const int e = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (e >= n) return;  // wave-uniform
  const double tau = qb_read_wave(pooled, nbins, (long long)k, (long long)n);
  const double q = qb_read_wave(hist + (int64_t)e * nbins, nbins, (long long)k, (long long)n);
  if (tau != tau || q != q) return;
  if ((threadIdx.x & 63) == 0) bias[e] = (float)(tau - q);
}

}  // namespace lmoe
