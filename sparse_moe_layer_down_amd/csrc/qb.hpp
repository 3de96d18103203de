// Quantile Balancing kernels ("Kimi K3 Architecture Deep Dive" §3: scores in
// [0,1], a fixed B-bin histogram per expert, histograms summed across devices,
// the quantile read from the sum; "Inside K3" section Quantile Balancing;
// LeiPhone report "Keeping the numbers in range": each expert's threshold is
// moved to where it gets its target share).
//
//   qb_hist_kernel   LDS-privatised histogram: a work-group owns EG experts
//                    x a run of tokens, counts in LDS with ds atomics, then adds
//                    its non-zero bins to the global int32 histogram.
//   qb_pool_kernel   pooled histogram sum_e H[e] (int64), per expert slice, atomically summed.
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

// grid: (expert groups, token runs); dynamic LDS = eg * nbins * 4 bytes.
// When n and the group width are multiples of 4, each thread reads four
// adjacent experts of a token as one 16-B load and four tokens per iteration;
// otherwise one thread walks the group's experts of one token at a time.
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
  if ((n & 3) == 0 && (ne & 3) == 0) {
    const int nq = ne >> 2;            // 16-B quads per token
    const int rows = 256 / nq;          // tokens per pass
    const int tr = threadIdx.x / nq, q = threadIdx.x - tr * nq;
    if (tr < rows) {
      const float *base = scores + e0 + q * 4;
      int32_t *hq = h + q * 4 * nbins;
      int64_t t = t0 + tr;
      for (; t + 3 * rows < t1; t += 4 * rows) {
        f32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *(const f32x4 *)(base + (t + u * rows) * n);
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int c = 0; c < 4; ++c) atomicAdd(&hq[c * nbins + qb_bin(v[u][c], nbins)], 1);
      }
      for (; t < t1; t += rows) {
        const f32x4 v = *(const f32x4 *)(base + t * n);
#pragma unroll
        for (int c = 0; c < 4; ++c) atomicAdd(&hq[c * nbins + qb_bin(v[c], nbins)], 1);
      }
    }
  } else {
    for (int64_t t = t0 + threadIdx.x; t < t1; t += blockDim.x) {
      const float *row = scores + t * n + e0;
      for (int e = 0; e < ne; ++e) atomicAdd(&h[e * nbins + qb_bin(row[e], nbins)], 1);
    }
  }
  __syncthreads();
  if ((nbins & 1) == 0) {
    // two adjacent bins of one expert per 64-bit atomic: the pair is 8-byte
    // aligned (even bin, even row length, 16-byte aligned histogram) and the low
    // count cannot carry into the high one while both stay non-negative int32
    for (int i = 2 * threadIdx.x; i < ne * nbins; i += 2 * blockDim.x) {
      const uint32_t a = (uint32_t)h[i], b = (uint32_t)h[i + 1];
      if (a | b)
        atomicAdd((unsigned long long *)&hist[(int64_t)(e0 + i / nbins) * nbins + (i % nbins)],
                  ((unsigned long long)b << 32) | a);
    }
  } else {
    for (int i = threadIdx.x; i < ne * nbins; i += blockDim.x) {
      const int v = h[i];
      if (v) atomicAdd(&hist[(int64_t)(e0 + i / nbins) * nbins + (i % nbins)], v);
    }
  }
}

// pooled[j] = sum_e hist[e][j]: grid (bin chunks of 64, expert slices); a
// block of 256 threads = 64 bins x 4 expert stripes sums its slice and adds it
// to pooled (zeroed beforehand) with one 64-bit atomic per bin.
constexpr int QB_POOL_SLICE = 64;  // experts per block
__global__ __launch_bounds__(256) void qb_pool_kernel(const int32_t *__restrict__ hist, int n, int nbins,
                                                      unsigned long long *__restrict__ pooled) {
  __shared__ long long part[4][64];
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  const int stripe = threadIdx.x >> 6;
  const int ea = blockIdx.y * QB_POOL_SLICE, eb = min(n, ea + QB_POOL_SLICE);
  long long s = 0;
  if (j < nbins)
    for (int e = ea + stripe; e < eb; e += 4) s += hist[(int64_t)e * nbins + j];
  part[stripe][threadIdx.x & 63] = s;
  __syncthreads();
  if (stripe == 0 && j < nbins) {
    const long long v = part[0][threadIdx.x] + part[1][threadIdx.x] + part[2][threadIdx.x] + part[3][threadIdx.x];
    if (v) atomicAdd(&pooled[j], (unsigned long long)v);
  }
}

__global__ void fill_u64_kernel(unsigned long long *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
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
                                                       const unsigned long long *__restrict__ pooled, int n, int nbins,
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
