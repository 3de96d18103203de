// Quantile Balancing kernels ("Kimi K3 Architecture Deep Dive" §3: scores in
// [0,1], a fixed B-bin histogram per expert, histograms summed across devices,
// the quantile read from the sum; "Inside K3" section Quantile Balancing;
// LeiPhone report "Keeping the numbers in range": each expert's threshold is
// moved to where it gets its target share).
//
//   qb_hist_kernel   LDS-privatised histogram: a work-group owns EG experts
//                    x a run of tokens and counts in LDS with ds atomics; with
//                    one run it writes (or adds) its bins to the histogram,
//                    with several it stores them to its run's slab.
//   qb_merge_kernel  histogram (or histogram +) = the runs' slabs summed in order.
//   qb_merge_pool_kernel  the same merge, also summing the pooled histogram (used
//                    when the update solves).
//   qb_pool_kernel   pooled histogram sum_e H[e] (int64), per expert slice, atomically summed.
//   qb_solve_wide_kernel  the same solve for histograms of more than 1024
//                    bins, each expert's bins staged in LDS, tau read once by an
//                    extra work-group, the bias written by the last one to finish
//   qb_solve_kernel  one wavefront per expert: tail sums G(j) by a wave scan,
//                    j* = max{j : G(j) >= c}, q by linear interpolation inside
//                    bin j*, bias = fp32(tau - q) with tau read the same way
//                    from the pooled histogram (by one more wave of the
//                    work-group, beside the experts' reads).  All counts are integers and
//                    the interpolation is the same sequence of IEEE fp64
//                    operations as the definition, so the result is exact.
//
// The margin form of the estimator ("Keeping the numbers in range": read the
// scores against the top-k threshold and solve where each expert's threshold
// must move):
//   qb_thresholds_kernel  one wavefront per token: the k-th and (k+1)-th
//                         largest selection keys s + b (k + 1 rounds of a wave
//                         maximum, as in the top-k kernel)
//   qb_hist_kernel<true>  histogram of each (token, expert) margin against the
//                         threshold that expert must cross, mapped to [0,1]
//   qb_margin_solve_kernel  b_e -= (2 q_e - 1), q_e read as above
// and the K2-style fixed-step baseline the pages compare QB with:
//   signsgd_kernel        per-expert loads from the top-k lists, then
//                         b_e += step * sign(T k / n - load_e)
#pragma once
#include "common.hpp"
#include "route.hpp"

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

// The value the margin form bins for score s of an expert with bias b in a
// token whose k-th / (k+1)-th largest keys are tk / tk1: the key sel = s + b,
// its margin against the threshold it must cross (tk1 if it is at or above tk,
// else tk), mapped to [0,1] as (m + 1) / 2.  Every step is one fp32 operation
// (no contraction), so the host can reproduce it exactly.
LMOE_DEV float qb_margin_u(float s, float b, float tk, float tk1) {
#pragma clang fp contract(off)
  const float sel = s + b;
  const float m = sel - (sel >= tk ? tk1 : tk);
  return (m + 1.0f) * 0.5f;
}

// One work-group per (token run r, expert group g), walked through a 1-D grid
// of 8 * ceil(groups * runs / 8) work-groups: work item w = r * groups + g, and
// XCD x (work-groups are dispatched round-robin over the 8 XCDs) takes items
// [x * chunk, (x + 1) * chunk) in order, so neighbouring expert groups of one
// run, which read the same 128-byte lines of the score rows, share an L2.
// Dynamic LDS = eg * nbins * 4 bytes.  QUAD (n and the group width multiples
// of 4): each thread reads four adjacent experts of a token as one 16-B load,
// in batches of tokens (the kernel is bound by these strided loads, not by the
// LDS atomics, so it keeps many in flight); otherwise one thread walks the
// group's experts of one token at a time.  (Two instantiations, so that each
// path gets its own register allocation and occupancy.)
// Output: with runs == 1 the group's bins go to hist (stored, or added when
// accumulate != 0: every bin of the group belongs to this work-group alone);
// with runs > 1 to part[r][e][bin], summed by qb_merge_kernel (or qb_merge_pool_kernel).
// MARGIN: bin qb_margin_u of the score (bias [n], thr [T] = {tk, tk1}) instead
// of the score itself.  pooled (may be null): nbins counters that work-group 0
// zeroes for a later qb_merge_pool_kernel.  slab16: the runs' slabs hold 16-bit
// counts (a run has fewer than 65536 tokens; n * nbins and the group width are
// multiples of 8, so each group's counts start 16-byte aligned).
constexpr int QB_HIST_THREADS = 512;
// The pooled histogram's nbins counters are followed by tau (a double) and the
// wide solve's completion counter, zeroed with the counters.
constexpr int QB_POOLED_EXTRA = 2;
constexpr int QB_MAX_RUNS = 16;  // token runs of one histogram launch (slabs in the workspace)

template <bool MARGIN, bool QUAD>
__global__ __launch_bounds__(QB_HIST_THREADS) void qb_hist_kernel(const float *__restrict__ scores, int64_t T, int n,
                                                      int nbins, int eg, int groups, int runs,
                                                      int64_t tokens_per_block, int32_t *__restrict__ hist,
                                                      int32_t *__restrict__ part, int accumulate,
                                                      const float *__restrict__ bias,
                                                      const float2 *__restrict__ thr,
                                                      unsigned long long *__restrict__ pooled, int slab16) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  int32_t *h = (int32_t *)smem_raw;
  const int items = groups * runs;
  const int chunk = (items + 7) / 8;
  const int w = (int)(blockIdx.x % 8) * chunk + (int)(blockIdx.x / 8);
  if (w >= items) return;  // uniform over the work-group, before any barrier
  if (pooled && blockIdx.x == 0)
    for (int i = threadIdx.x; i < nbins + QB_POOLED_EXTRA; i += blockDim.x) pooled[i] = 0ull;
  const int run = w / groups, g = w - run * groups;
  const int e0 = g * eg;
  const int ne = min(eg, n - e0);
  for (int i = threadIdx.x; i < ne * nbins; i += blockDim.x) h[i] = 0;
  __syncthreads();
  const int64_t t0 = (int64_t)run * tokens_per_block;
  const int64_t t1 = min(T, t0 + tokens_per_block);
  if constexpr (QUAD) {  // 16-byte aligned quads (ne and e0 are multiples of 4 too)
    constexpr int U = 4;                // tokens per thread and batch
    const int nq = ne >> 2;            // 16-B quads per token
    const int rows = QB_HIST_THREADS / nq;  // tokens per pass
    const int tr = threadIdx.x / nq, q = threadIdx.x - tr * nq;
    if (tr < rows) {
      const float *base = scores + e0 + q * 4;
      int32_t *hq = h + q * 4 * nbins;
      f32x4 bq = {0.0f, 0.0f, 0.0f, 0.0f};
      if (MARGIN) bq = *(const f32x4 *)(bias + e0 + q * 4);
      // Batches of U tokens (rows apart) alternate between two register sets:
      // the loads of the next batch are issued before the atomics of the
      // current one, and a short last batch is masked rather than walked a
      // token at a time, so a run costs about one memory latency per batch.
      const int64_t step = (int64_t)U * rows;
      f32x4 va[U], vb[U];
      float2 tha[U], thb[U];
      auto load = [&](int64_t tb, f32x4 (&v)[U], float2 (&th)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t t = tb + (int64_t)u * rows;
          if (t < t1) {
            v[u] = *(const f32x4 *)(base + t * n);
            if (MARGIN) th[u] = thr[t];
          }
        }
      };
      auto count = [&](int64_t tb, const f32x4 (&v)[U], const float2 (&th)[U]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (tb + (int64_t)u * rows < t1) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float x = MARGIN ? qb_margin_u(v[u][c], bq[c], th[u].x, th[u].y) : v[u][c];
              atomicAdd(&hq[c * nbins + qb_bin(x, nbins)], 1);
            }
          }
      };
      int64_t tb = t0 + tr;
      if (tb < t1) load(tb, va, tha);
      while (tb < t1) {
        if (tb + step < t1) load(tb + step, vb, thb);
        count(tb, va, tha);
        tb += step;
        if (tb >= t1) break;
        if (tb + step < t1) load(tb + step, va, tha);
        count(tb, vb, thb);
        tb += step;
      }
    }
  } else {
    constexpr int U = 4;  // tokens per thread and iteration
    const int64_t bd = blockDim.x;
    int64_t t = t0 + threadIdx.x;
    for (; t + (U - 1) * bd < t1; t += U * bd) {
      float2 th[U];
#pragma unroll
      for (int u = 0; u < U; ++u) th[u] = MARGIN ? thr[t + u * bd] : float2{0.0f, 0.0f};
      for (int e = 0; e < ne; ++e) {
        float x[U];
#pragma unroll
        for (int u = 0; u < U; ++u) x[u] = scores[(t + u * bd) * n + e0 + e];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float y = MARGIN ? qb_margin_u(x[u], bias[e0 + e], th[u].x, th[u].y) : x[u];
          atomicAdd(&h[e * nbins + qb_bin(y, nbins)], 1);
        }
      }
    }
    for (; t < t1; t += bd) {
      const float *row = scores + t * n + e0;
      float2 th = {0.0f, 0.0f};
      if (MARGIN) th = thr[t];
      for (int e = 0; e < ne; ++e) {
        const float x = MARGIN ? qb_margin_u(row[e], bias[e0 + e], th.x, th.y) : row[e];
        atomicAdd(&h[e * nbins + qb_bin(x, nbins)], 1);
      }
    }
  }
  __syncthreads();
  // the group's bins are contiguous ([e0, e0 + ne) x nbins) in hist and in the slab
  const int64_t off = (int64_t)e0 * nbins;
  const int cnt = ne * nbins;
  if (runs > 1 && slab16) {  // eight counts per 16-byte store
    uint16_t *dst = (uint16_t *)part + (int64_t)run * n * nbins + off;
    const int c8 = cnt / 8;
    for (int i = threadIdx.x; i < c8; i += blockDim.x) {
      const int4 a = *(const int4 *)(h + 8 * i), b = *(const int4 *)(h + 8 * i + 4);
      *(u32x4 *)(dst + 8 * i) = u32x4{(uint32_t)a.x | ((uint32_t)a.y << 16), (uint32_t)a.z | ((uint32_t)a.w << 16),
                                      (uint32_t)b.x | ((uint32_t)b.y << 16), (uint32_t)b.z | ((uint32_t)b.w << 16)};
    }
    for (int i = 8 * c8 + threadIdx.x; i < cnt; i += blockDim.x) dst[i] = (uint16_t)h[i];
  } else if (runs > 1) {
    int32_t *dst = part + (int64_t)run * n * nbins + off;
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) dst[i] = h[i];
  } else if (accumulate) {
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) hist[off + i] += h[i];
  } else {
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) hist[off + i] = h[i];
  }
}

// hist[i] = (accumulate ? hist[i] : 0) + sum over r < runs of part[r][i], r in
// order; one element per thread, the runs' loads issued together.  SL: the slab
// element type (int32_t, or uint16_t for 16-bit slabs).
template <typename SL>
__global__ __launch_bounds__(256) void qb_merge_kernel(const SL *__restrict__ part, int runs, int64_t cnt,
                                                       int32_t *__restrict__ hist, int accumulate) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cnt) return;
  int32_t v[QB_MAX_RUNS];
#pragma unroll
  for (int r = 0; r < QB_MAX_RUNS; ++r) v[r] = r < runs ? (int32_t)part[r * cnt + i] : 0;
  int32_t s = accumulate ? hist[i] : 0;
#pragma unroll
  for (int r = 0; r < QB_MAX_RUNS; ++r) s += v[r];
  hist[i] = s;
}

// The merge of several runs' slabs fused with the pooled sum:
//   hist[e][j] = (accumulate ? hist[e][j] : 0) + sum over runs r (in order) of part[r][e][j]
//   pooled[j] += sum over the block's experts e of the new hist[e][j]
// (pooled zeroed beforehand).  Grid (bin chunks of 64, expert slices of
// QB_MP_SLICE); a block of 256 threads = 64 bins x 4 expert stripes sums its
// slice and adds it to pooled with one 64-bit atomic per bin.
constexpr int QB_MP_SLICE = 16;
template <typename SL>
__global__ __launch_bounds__(256) void qb_merge_pool_kernel(const SL *__restrict__ part, int runs, int n,
                                                            int nbins, int32_t *__restrict__ hist, int accumulate,
                                                            unsigned long long *__restrict__ pooled) {
  __shared__ long long red[4][64];
  const int lane = threadIdx.x & 63, stripe = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const int ea = blockIdx.y * QB_MP_SLICE, eb = min(n, ea + QB_MP_SLICE);
  const int64_t cnt = (int64_t)n * nbins;
  long long s = 0;
  if (j < nbins) {
#pragma unroll
    for (int i = 0; i < QB_MP_SLICE / 4; ++i) {
      const int e = ea + stripe + 4 * i;
      if (e < eb) {
        const int64_t idx = (int64_t)e * nbins + j;
        int32_t v[QB_MAX_RUNS];
#pragma unroll
        for (int r = 0; r < QB_MAX_RUNS; ++r) v[r] = r < runs ? (int32_t)part[r * cnt + idx] : 0;
        int32_t hv = accumulate ? hist[idx] : 0;
#pragma unroll
        for (int r = 0; r < QB_MAX_RUNS; ++r) hv += v[r];
        hist[idx] = hv;
        s += hv;
      }
    }
  }
  red[stripe][lane] = s;
  __syncthreads();
  if (stripe == 0 && j < nbins) {
    const long long v = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    if (v) atomicAdd(&pooled[j], (unsigned long long)v);
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
  if (j < nbins) {
    int32_t v[QB_POOL_SLICE / 4];
#pragma unroll
    for (int i = 0; i < QB_POOL_SLICE / 4; ++i) {
      const int e = ea + stripe + 4 * i;
      v[i] = e < eb ? hist[(int64_t)e * nbins + j] : 0;
    }
#pragma unroll
    for (int i = 0; i < QB_POOL_SLICE / 4; ++i) s += v[i];
  }
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

// Upper-tail read of one histogram by a full wavefront: lane l owns bins
// [l * per, (l + 1) * per), per = ceil(nbins / 64).  Returns q, or a NaN when
// the histogram is empty.  c = N * k / n where N is the histogram's mass.
// Up to QB_LANE_BINS bins per lane (nbins <= 1024) a lane's bins are first
// loaded into registers (all loads in flight at once) and both passes use that
// copy; wider histograms are read in chunks of QB_LANE_BINS bins, each chunk's
// loads issued together.  Both forms perform the same sequence of integer and
// fp64 operations as a bin-by-bin walk.
constexpr int QB_LANE_BINS = 16;

template <typename CT>
LMOE_DEV void qb_lane_load(const CT *h, int nbins, long long (&v)[QB_LANE_BINS]) {
  const int per = (nbins + 63) / 64;
  const int lo = min((int)(threadIdx.x & 63) * per, nbins), hi = min(lo + per, nbins);
#pragma unroll
  for (int i = 0; i < QB_LANE_BINS; ++i) v[i] = lo + i < hi ? (long long)h[lo + i] : 0;
}

// CACHED: v holds the lane's bins (qb_lane_load); otherwise h is read.
template <bool CACHED, typename CT>
LMOE_DEV double qb_read_wave(const CT *h, const long long (&v)[QB_LANE_BINS], int nbins, long long k, long long n) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x & 63;
  const int per = (nbins + 63) / 64;
  const int lo = min(lane * per, nbins), hi = min(lo + per, nbins);
  long long mine = 0;
  if (CACHED) {
#pragma unroll
    for (int i = 0; i < QB_LANE_BINS; ++i) mine += v[i];
  } else {  // chunks of QB_LANE_BINS bins, each chunk's loads in flight together
    for (int j0 = lo; j0 < hi; j0 += QB_LANE_BINS) {
      long long w[QB_LANE_BINS];
#pragma unroll
      for (int i = 0; i < QB_LANE_BINS; ++i) w[i] = j0 + i < hi ? (long long)h[j0 + i] : 0;
#pragma unroll
      for (int i = 0; i < QB_LANE_BINS; ++i) mine += w[i];
    }
  }
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
  // the highest bin j of my range with G(j) >= c
  if (CACHED) {
    bool found = false;
#pragma unroll
    for (int i = QB_LANE_BINS - 1; i >= 0; --i) {
      if (!found && lo + i < hi) {
        const long long gj = G + v[i];
        if ((double)gj >= c) {
          jcand = lo + i;
          Gnext = G;
          hj = v[i];
          found = true;
        } else {
          G = gj;
        }
      }
    }
  } else {
    // Only the range that holds j* needs the walk: it is the highest non-empty
    // lane range whose bottom bin has G(lo) = incl >= c (G does not increase
    // with j, and G(0) = N >= c).  That range is split over the wave (a few
    // bins per lane), tail sums are taken across the lanes again, and each lane
    // walks its piece from the top as above.
    const unsigned long long holds = __ballot(lo < hi && (double)incl >= c);
    const int ol = 63 - __clzll((long long)holds);
    const int olo = __shfl(lo, ol, 64), ohi = __shfl(hi, ol, 64);
    const long long otop = __shfl(G, ol, 64);  // G(ohi)
    const int pp = (ohi - olo + 63) / 64;
    const int plo = min(olo + lane * pp, ohi), phi = min(plo + pp, ohi);
    long long part = 0;
    for (int j = plo; j < phi; ++j) part += (long long)h[j];
    long long pin = part;  // inclusive suffix scan of the pieces (lanes >= me)
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long other = __shfl_down(pin, o, 64);
      if (lane + o < 64) pin += other;
    }
    long long Gp = otop + (pin - part);  // G(phi)
    for (int j = phi - 1; j >= plo; --j) {
      const long long hv = (long long)h[j];
      const long long gj = Gp + hv;
      if ((double)gj >= c) {
        jcand = j;
        Gnext = Gp;
        hj = hv;
        break;
      }
      Gp = gj;
    }
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

// Histograms of up to 64 * QB_LANE_BINS bins.  A work-group of five waves:
// waves 0-3 read q of experts 4 * blockIdx.x + w, wave 4 reads tau from the
// pooled histogram at the same time (the two reads overlap instead of running
// one after the other in each wave), then waves 0-3 write fp32(tau - q).
constexpr int QB_SOLVE_EXPERTS = 4;  // experts per work-group (plus one wave for tau)
__global__ __launch_bounds__(64 * (QB_SOLVE_EXPERTS + 1)) void qb_solve_kernel(
    const int32_t *__restrict__ hist, const unsigned long long *__restrict__ pooled, int n, int nbins, int k,
    float *__restrict__ bias) {
#pragma clang fp contract(off)
  __shared__ double s_tau;
  const int w = threadIdx.x >> 6;
  const int e = blockIdx.x * QB_SOLVE_EXPERTS + w;
  long long v[QB_LANE_BINS];
  double r = 0.0;
  if (w == QB_SOLVE_EXPERTS) {
    qb_lane_load(pooled, nbins, v);
    r = qb_read_wave<true>(pooled, v, nbins, (long long)k, (long long)n);
    if ((threadIdx.x & 63) == 0) s_tau = r;
  } else if (e < n) {
    const int32_t *he = hist + (int64_t)e * nbins;
    qb_lane_load(he, nbins, v);
    r = qb_read_wave<true>(he, v, nbins, (long long)k, (long long)n);
  }
  __syncthreads();
  if (w == QB_SOLVE_EXPERTS || e >= n) return;
  const double tau = s_tau;
  if (tau != tau || r != r) return;
  if ((threadIdx.x & 63) == 0) bias[e] = (float)(tau - r);
}

// Histograms wider than a lane's register copy (nbins > 64 * QB_LANE_BINS):
// qb_solve_wide_kernel (below) gives each expert one wave that stages the
// expert's histogram in its own LDS region (coalesced loads) before reading q,
// and one more work-group that stages the pooled histogram and reads tau; the
// reads are those of qb_read_wave, so the bias is the same bits as
// qb_solve_kernel's.
// Copies `count` 4- or 8-byte counters from global memory to LDS with `nth`
// threads (this one is `id`): 16-byte loads when both sides are 16-byte
// aligned, each thread's loads of a batch (up to B of them) issued before any
// of its LDS stores, so a batch costs one memory latency.
template <int B, typename E>
LMOE_DEV void qb_stage_lds(E *dst, const E *__restrict__ src, int count, int id, int nth) {
  constexpr int PER = 16 / (int)sizeof(E);
  int done = 0;
  if ((((uintptr_t)src | (uintptr_t)dst) & 15) == 0) {
    const int nv = count / PER;
    const u32x4 *s4 = (const u32x4 *)src;
    u32x4 *d4 = (u32x4 *)dst;
    for (int i0 = id; i0 < nv; i0 += B * nth) {
      u32x4 r[B];
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (i0 + u * nth < nv) r[u] = s4[i0 + u * nth];
#pragma unroll
      for (int u = 0; u < B; ++u)
        if (i0 + u * nth < nv) d4[i0 + u * nth] = r[u];
    }
    done = nv * PER;
  }
  for (int i0 = done + id; i0 < count; i0 += B * nth) {
    E r[B];
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (i0 + u * nth < count) r[u] = src[i0 + u * nth];
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (i0 + u * nth < count) dst[i0 + u * nth] = r[u];
  }
}

// Work-groups 0 .. gridDim.x - 2: wpb waves, wave w reads q of expert
// blockIdx.x * wpb + w from its own LDS region of nbins counters and stores it
// to qv[e]; the last work-group stages the pooled histogram in LDS (nbins
// 64-bit counters) and its wave 0 reads tau into *tau.  Each work-group then
// counts itself done (*done, zero at launch); the last one to finish writes
// bias[e] = fp32(tau - q_e) for every expert, so tau is read beside the q reads
// instead of by a launch before them.  No work-group waits for another.
// Dynamic LDS: flag_off = max(wpb * nbins * 4, nbins * 8) bytes of staging,
// then one word.
__global__ __launch_bounds__(256) void qb_solve_wide_kernel(const int32_t *__restrict__ hist,
                                                            const unsigned long long *__restrict__ pooled,
                                                            double *__restrict__ tau, unsigned int *__restrict__ done,
                                                            double *__restrict__ qv, int n, int nbins, int k, int wpb,
                                                            int flag_off, float *__restrict__ bias) {
#pragma clang fp contract(off)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  int &s_last = *(int *)(smem_raw + flag_off);  // one LDS word past the staging regions
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  long long v[QB_LANE_BINS];
  if (blockIdx.x == gridDim.x - 1) {
    unsigned long long *hp = (unsigned long long *)smem_raw;
    qb_stage_lds<8>(hp, pooled, nbins, (int)threadIdx.x, (int)blockDim.x);
    __syncthreads();
    if (w == 0) {
      const double t = qb_read_wave<false>(hp, v, nbins, (long long)k, (long long)n);
      if (lane == 0) *tau = t;
    }
  } else {
    const int e = blockIdx.x * wpb + w;
    if (e < n) {  // wave-uniform
      int32_t *mine = (int32_t *)smem_raw + (int64_t)w * nbins;
      qb_stage_lds<16>(mine, hist + (int64_t)e * nbins, nbins, lane, 64);
      // the wave reads bins other lanes wrote: its LDS writes complete first
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      const double q = qb_read_wave<false>(mine, v, nbins, (long long)k, (long long)n);
      if (lane == 0) qv[e] = q;
    }
  }
  __syncthreads();  // this work-group's stores precede its count
  if (threadIdx.x == 0) {
    __threadfence();
    s_last = atomicAdd(done, 1u) == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;  // uniform over the work-group
  __threadfence();      // every other work-group's stores are visible from here
  const double t = *(volatile const double *)tau;
  for (int e = threadIdx.x; e < n; e += blockDim.x) {
    const double q = *(volatile const double *)(qv + e);
    if (t == t && q == q) bias[e] = (float)(t - q);
  }
}

// Inverse of ord_f32 (for keys that came from a float): the float whose
// order-preserving bits are u.
LMOE_DEV float unord_f32(uint32_t u) {
  return __builtin_bit_cast(float, (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// One wavefront per token: tk = the k-th and tk1 = the (k+1)-th largest of the
// n keys s + b (tk1 = -inf when k == n), selected as by the top-k kernel
// (wave_topk, which keys order the same way) but in its values-only form.
template <int MAXJ>
__global__ __launch_bounds__(256) void qb_thresholds_kernel(const float *__restrict__ s,
                                                            const float *__restrict__ bias, int T, int n, int k,
                                                            float2 *__restrict__ thr) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  const int rounds = min(k + 1, n);
  for (int t = wave; t < T; t += nwaves) {
    uint32_t hi[MAXJ];
    token_keys<MAXJ>(s + (int64_t)t * n, bias, n, hi);
    float tk = 0.0f, tk1 = -INFINITY;
    wave_topk<MAXJ, true>(hi, rounds, [&](int r, uint64_t g) {
      const float v = unord_f32((uint32_t)(g >> 32));
      if (r == k - 1) tk = v;
      if (r == k) tk1 = v;
    });
    if (lane == 0) thr[t] = make_float2(tk, tk1);
  }
}

// Margin solve: one wavefront per expert; b_e <- fp32(b_e - (2 q_e - 1)) in
// fp64, where q_e is the upper-(k/n) read of the expert's margin histogram.
// Experts with an empty histogram keep their bias.
__global__ __launch_bounds__(256) void qb_margin_solve_kernel(const int32_t *__restrict__ hist, int n, int nbins,
                                                              int k, float *__restrict__ bias) {
#pragma clang fp contract(off)
  const int e = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  if (e >= n) return;  // wave-uniform
  const int32_t *he = hist + (int64_t)e * nbins;
  long long vh[QB_LANE_BINS];
  double q;
  if (nbins <= 64 * QB_LANE_BINS) {
    qb_lane_load(he, nbins, vh);
    q = qb_read_wave<true>(he, vh, nbins, (long long)k, (long long)n);
  } else {
    q = qb_read_wave<false>(he, vh, nbins, (long long)k, (long long)n);
  }
  if (q != q) return;
  if ((threadIdx.x & 63) == 0) bias[e] = (float)((double)bias[e] - (2.0 * q - 1.0));
}

// SignSGD-style step: work-group g counts the loads of experts 256 g .. + 255
// over all T k top-k entries (LDS counters), then
//   bias[e] += step * sign(T k - load_e * n)
// (the comparison with the share T k / n is exact in integers; one fp32 add).
__global__ __launch_bounds__(1024) void signsgd_kernel(const int32_t *__restrict__ idx, int64_t entries, int n,
                                                       float step, float *__restrict__ bias) {
  __shared__ int32_t cnt[256];
  const int e0 = blockIdx.x * 256;
  if (threadIdx.x < 256) cnt[threadIdx.x] = 0;
  __syncthreads();
  for (int64_t i = threadIdx.x; i < entries; i += blockDim.x) {
    const unsigned r = (unsigned)(idx[i] - e0);
    if (r < 256u) atomicAdd(&cnt[r], 1);
  }
  __syncthreads();
  const int e = e0 + (int)threadIdx.x;
  if (threadIdx.x < 256 && e < n) {
    const long long load = (long long)cnt[threadIdx.x] * n;
    const float sg = entries > load ? step : (entries < load ? -step : 0.0f);
    bias[e] = bias[e] + sg;
  }
}

}  // namespace lmoe
