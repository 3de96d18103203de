// Router top-k and token permutation kernels.
//
// Top-k ("Kimi K3 Architecture Deep Dive" §3: 896-choose-16 with a loss-free
// selection bias; LeiPhone report "Keeping the numbers in range": the bias
// steers selection): one wavefront per token.  Lane l holds experts
// l, l+64, ... as 64-bit keys (order-preserving bits of s+b, then the
// complemented expert index), so a single max-reduction picks the largest
// biased score and, among equal scores, the lowest index.  k rounds of
// "local max -> wave max -> winner drops it" give the k largest without
// sorting the n scores.  Routing weights renormalise the unbiased scores of
// the chosen experts.
//
// Permutation (dispatch of tokens to experts, rows ordered by expert then
// token): tokens are cut into chunks of 256.  For each chunk and expert a
// 256-bit mask of the tokens that chose the expert is built in LDS; a single
// scan work-group turns mask popcounts into per-(chunk, expert) prefixes and the
// global expert offsets, and writes the grouped-GEMM tile table; the scatter
// kernel then places (token, slot) at expert offset + prefix + popcount(mask
// bits below the token).  Every step is integer and deterministic.
#pragma once
#include "common.hpp"

namespace lmoe {

constexpr int PERM_CHUNK = 256;  // tokens per permutation chunk (4 mask words)
constexpr int SCHED_COUNTERS = 8;  // tile counters per grouped GEMM launch (one per XCD)

LMOE_DEV uint32_t ord_f32(float f) {
  f = f + 0.0f;  // -0 -> +0
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0u;  // NaN ranks lowest
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Maximum over the wavefront of 32-bit values, returned wave-uniform: DPP within
// each row of 16 lanes (swap neighbours, swap pairs, mirror halves, mirror the
// row), then the four row maxima through scalar lane reads.
template <int CTRL>
LMOE_DEV uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
LMOE_DEV uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));
  v = max(v, dpp_u32<0x4E>(v));
  v = max(v, dpp_u32<0x141>(v));
  v = max(v, dpp_u32<0x140>(v));
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}

// Maximum over the wavefront of the 64-bit keys (score word << 32 | index
// word): the maximum of the score words, then the index word of the one lane
// holding it; only when lanes tie on the score word is the maximum of their
// index words taken.
LMOE_DEV uint64_t wave_max_key(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  const uint32_t mh = wave_max_u32(hi);
  const uint64_t holders = __ballot(hi == mh);
  uint32_t ml;
  if (__popcll(holders) == 1)
    ml = (uint32_t)__builtin_amdgcn_readlane((int)lo, __ffsll((long long)holders) - 1);
  else
    ml = wave_max_u32(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// The k largest keys of one token, one wavefront: lane l holds experts
// e = l + 64 j (j < MAXJ) as the score words hi[j] = ord_f32(s_e + b_e) (0 for
// e >= n); the full key of e is (hi << 32) | ~e, so the larger biased score wins
// and, among equal scores, the lower index.  The index half follows from the lane
// and the slot, so a lane keeps only the score words and compares 32-bit words.
// visit(r, g) receives the r-th largest key g, r = 0 .. rounds - 1.  Each lane
// caches its two largest remaining keys; keys are unique and a lane's wins come
// in decreasing order, so its remaining keys are exactly those below its last
// win, and when the cache runs out (a lane's second, fourth, ... win) it rescans
// for the two largest keys below that win (no key is ever cleared).
// VALUES: only the score words of the r-th largest keys are wanted (the k-th
// largest value, counted with multiplicity, does not depend on which of several
// equal keys is taken), so a round takes the 32-bit maximum alone and the lowest
// lane holding it drops one key; visit then receives the word in the high half.
template <int MAXJ, bool VALUES = false, typename F>
LMOE_DEV void wave_topk(const uint32_t (&hi)[MAXJ], int rounds, F &&visit) {
  const int lane = threadIdx.x & 63;
  uint32_t bh = 0, sh = 0;  // best and second remaining key of this lane: score word, slot
  int bj = -1, sj = -1;     // (slot < 0: none)
  auto top2_below = [&](uint32_t lh, int lj) {  // keys (h, j) below (lh, lj) in key order
    bh = 0;
    sh = 0;
    bj = -1;
    sj = -1;
#pragma unroll
    for (int j = 0; j < MAXJ; ++j) {
      const uint32_t h = hi[j];
      const bool ok = h < lh || (h == lh && j > lj);
      // slots ascend, so an equal score word never beats an earlier slot
      const bool gb = ok && (bj < 0 || h > bh);
      const bool gs = ok && !gb && (sj < 0 || h > sh);
      sh = gb ? bh : (gs ? h : sh);
      sj = gb ? bj : (gs ? j : sj);
      bh = gb ? h : bh;
      bj = gb ? j : bj;
    }
  };
  top2_below(0xFFFFFFFFu, -1);  // every key (no score word reaches all ones)
  for (int r = 0; r < rounds; ++r) {
    bool drop;
    if constexpr (VALUES) {
      const uint32_t mh = wave_max_u32(bj >= 0 ? bh : 0u);
      const uint64_t holders = __ballot(bj >= 0 && bh == mh);
      visit(r, (uint64_t)mh << 32);
      drop = lane == __ffsll((long long)holders) - 1;
    } else {
      const uint64_t mine = bj >= 0 ? ((uint64_t)bh << 32) | (0xFFFFFFFFu - (uint32_t)(lane + 64 * bj)) : 0ull;
      const uint64_t g = wave_max_key(mine);
      visit(r, g);
      drop = bj >= 0 && mine == g;
    }
    if (drop) {  // the owning lane drops the winner
      if (sj >= 0) {
        bh = sh;
        bj = sj;
        sj = -1;
      } else {
        top2_below(bh, bj);
      }
    }
  }
}

// The score words of a token's keys (see wave_topk): s + b of expert
// lane + 64 j, loads issued together (padding slots load nothing).
template <int MAXJ>
LMOE_DEV void token_keys(const float *row, const float *bias, int n, uint32_t (&hi)[MAXJ]) {
  const int lane = threadIdx.x & 63;
  float sv[MAXJ], bv[MAXJ];
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) {
    const int e = lane + 64 * j;
    sv[j] = e < n ? row[e] : 0.0f;
    bv[j] = e < n ? bias[e] : 0.0f;
  }
#pragma unroll
  for (int j = 0; j < MAXJ; ++j) hi[j] = lane + 64 * j < n ? ord_f32(sv[j] + bv[j]) : 0u;
}

template <int MAXJ>
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ s, const float *__restrict__ bias,
                                                   int T, int n, int k, int32_t *__restrict__ idx_out,
                                                   float *__restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * blockDim.x) >> 6;
  for (int t = wave; t < T; t += nwaves) {
    const float *row = s + (int64_t)t * n;
    uint32_t hi[MAXJ];
    token_keys<MAXJ>(row, bias, n, hi);
    int my_e = 0;
    wave_topk<MAXJ>(hi, k, [&](int r, uint64_t g) {
      if (lane == r) my_e = (int)(0xFFFFFFFFu - (uint32_t)g);
    });
    const float sv = lane < k ? row[my_e] : 0.0f;
    const float tot = wave_sum(sv);
    if (lane < k) {
      idx_out[(int64_t)t * k + lane] = my_e;
      w_out[(int64_t)t * k + lane] = sv / tot;
    }
  }
}

// masks[chunk][e][4] (uint64), ccount[chunk][e] (int32)
__global__ __launch_bounds__(256) void perm_mask_kernel(const int32_t *__restrict__ idx, int T, int n, int k,
                                                        uint64_t *__restrict__ masks,
                                                        int32_t *__restrict__ ccount) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  unsigned long long *m = (unsigned long long *)smem_raw;  // [n][4]
  const int c = blockIdx.x;
  for (int i = threadIdx.x; i < n * 4; i += blockDim.x) m[i] = 0ull;
  __syncthreads();
  const int tl = threadIdx.x;
  const int t = c * PERM_CHUNK + tl;
  if (t < T) {
    for (int r = 0; r < k; ++r) {
      const int e = idx[(int64_t)t * k + r];
      atomicOr(&m[e * 4 + (tl >> 6)], 1ull << (tl & 63));
    }
  }
  __syncthreads();
  uint64_t *gm = masks + (int64_t)c * n * 4;
  for (int i = threadIdx.x; i < n * 4; i += blockDim.x) gm[i] = m[i];
  for (int e = threadIdx.x; e < n; e += blockDim.x)
    ccount[(int64_t)c * n + e] = __popcll(m[e * 4]) + __popcll(m[e * 4 + 1]) + __popcll(m[e * 4 + 2]) +
                                 __popcll(m[e * 4 + 3]);
}

// Single work-group: each (chunk, expert) count replaced by the expert's rows in
// the chunks before it (the chunk's rows of expert e start at offs[e] plus
// that), the expert counts and offsets, and two grouped-GEMM tile tables
// (M-tile heights bm1 and bm2): entry j of a table is
// {expert, first row, end row} of one M tile.  The n_shared shared experts are
// appended as experts n .. n + n_shared - 1 whose rows are all T tokens (rows
// T*k + s*T .. + T, see perm_scatter_kernel); their tiles are interleaved
// evenly among the routed ones so that every contiguous range of the table
// (one XCD's share) gets the same mix.  ntiles[0], ntiles[1] = table lengths;
// ntiles[2 ..] = the grouped GEMMs' tile counters, zeroed here.
LMOE_DEV int interleave_pos(int i, bool shared, int nr, int ns, int q) {
  if (!shared) return i + min(i / q, ns);
  return (i + 1) * q <= nr ? (i + 1) * q + i : nr + i;
}
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t *__restrict__ cbase /* in: counts, out: prefixes */,
                                                         int nchunks, int n, int T, int k, int n_shared,
                                                         int32_t *__restrict__ counts, int32_t *__restrict__ offs,
                                                         int bm1, int4 *__restrict__ tiles1, int bm2,
                                                         int4 *__restrict__ tiles2, int32_t *__restrict__ ntiles) {
  __shared__ int32_t s_tot[1024];
  __shared__ int32_t s_t1[1024];
  __shared__ int32_t s_t2[1024];
  const int e = threadIdx.x;
  constexpr int CB = 16;  // chunk counts loaded together, so their latencies overlap
  int tot = 0;
  if (e < n) {
    for (int c0 = 0; c0 < nchunks; c0 += CB) {
      int v[CB];
#pragma unroll
      for (int j = 0; j < CB; ++j) v[j] = c0 + j < nchunks ? cbase[(int64_t)(c0 + j) * n + e] : 0;
#pragma unroll
      for (int j = 0; j < CB; ++j) {
        if (c0 + j < nchunks) cbase[(int64_t)(c0 + j) * n + e] = tot;
        tot += v[j];
      }
    }
  }
  const int t1 = (tot + bm1 - 1) / bm1, t2 = (tot + bm2 - 1) / bm2;
  s_tot[e] = e < n ? tot : 0;
  s_t1[e] = e < n ? t1 : 0;
  s_t2[e] = e < n ? t2 : 0;
  __syncthreads();
  // inclusive Hillis-Steele scans over 1024 entries
  for (int o = 1; o < 1024; o <<= 1) {
    const int a = e >= o ? s_tot[e - o] : 0;
    const int b = e >= o ? s_t1[e - o] : 0;
    const int c = e >= o ? s_t2[e - o] : 0;
    __syncthreads();
    s_tot[e] += a;
    s_t1[e] += b;
    s_t2[e] += c;
    __syncthreads();
  }
  if (e < 2 * SCHED_COUNTERS) ntiles[2 + e] = 0;  // the grouped GEMMs' tile counters start at zero
  const int R = T * k;  // routed rows; shared expert s owns rows R + s*T .. R + (s+1)*T
  const int nr1 = s_t1[1023], nr2 = s_t2[1023];
  const int mt1 = (T + bm1 - 1) / bm1, mt2 = (T + bm2 - 1) / bm2;
  const int ns1 = n_shared * mt1, ns2 = n_shared * mt2;
  const int q1 = ns1 > 0 ? max(1, nr1 / ns1) : 1, q2 = ns2 > 0 ? max(1, nr2 / ns2) : 1;
  if (e < n) {
    const int off = s_tot[e] - tot;
    counts[e] = tot;
    offs[e] = off;
    if (e == n - 1) {
      offs[n] = s_tot[e];
      ntiles[0] = nr1 + ns1;
      ntiles[1] = nr2 + ns2;
    }
    const int s1 = s_t1[e] - t1, s2 = s_t2[e] - t2;
    for (int j = 0; j < t1; ++j) {
      const int r0 = off + j * bm1;
      tiles1[interleave_pos(s1 + j, false, nr1, ns1, q1)] = make_int4(e, r0, min(r0 + bm1, off + tot), 0);
    }
    for (int j = 0; j < t2; ++j) {
      const int r0 = off + j * bm2;
      tiles2[interleave_pos(s2 + j, false, nr2, ns2, q2)] = make_int4(e, r0, min(r0 + bm2, off + tot), 0);
    }
  }
  for (int j = e; j < ns1; j += blockDim.x) {
    const int sh = j / mt1, r0 = R + sh * T + (j % mt1) * bm1;
    tiles1[interleave_pos(j, true, nr1, ns1, q1)] = make_int4(n + sh, r0, min(r0 + bm1, R + (sh + 1) * T), 0);
  }
  for (int j = e; j < ns2; j += blockDim.x) {
    const int sh = j / mt2, r0 = R + sh * T + (j % mt2) * bm2;
    tiles2[interleave_pos(j, true, nr2, ns2, q2)] = make_int4(n + sh, r0, min(r0 + bm2, R + (sh + 1) * T), 0);
  }
}

// Scatter (token, slot) to its dispatched row; also the shared experts' rows:
// row T*k + s*T + t is token t with weight 1 for shared expert s.  Grid: chunks
// x groups of four slots (the slots of a token are independent), so a few
// chunks still spread over many work-groups.
__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t *__restrict__ idx,
                                                           const float *__restrict__ w, int T, int n, int k,
                                                           int n_shared, const uint64_t *__restrict__ masks,
                                                           const int32_t *__restrict__ cbase,
                                                           const int32_t *__restrict__ offs,
                                                           int32_t *__restrict__ row_token,
                                                           float *__restrict__ row_w,
                                                           int32_t *__restrict__ slot_row) {
  const int c = blockIdx.x;
  const int tl = threadIdx.x;
  const int t = c * PERM_CHUNK + tl;
  if (t >= T) return;
  if (blockIdx.y == 0) {
    for (int sh = 0; sh < n_shared; ++sh) {
      const int64_t r = (int64_t)T * k + (int64_t)sh * T + t;
      row_token[r] = t;
      row_w[r] = 1.0f;
    }
  }
  const int wsel = tl >> 6;
  const uint64_t below = (1ull << (tl & 63)) - 1ull;
  // this work-group's four slots together, so their dependent loads (expert ->
  // mask words, base) overlap
  {
    const int r0 = 4 * blockIdx.y;
    int e[4], base[4];
    uint64_t mw[4][4];
    float wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = min(r0 + u, k - 1);
      e[u] = idx[(int64_t)t * k + r];
      wv[u] = w[(int64_t)t * k + r];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t *m = masks + ((int64_t)c * n + e[u]) * 4;
#pragma unroll
      for (int q = 0; q < 4; ++q) mw[u][q] = m[q];
      base[u] = offs[e[u]] + cbase[(int64_t)c * n + e[u]];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (r0 + u >= k) break;
      const uint64_t mine = wsel == 0 ? mw[u][0] : wsel == 1 ? mw[u][1] : wsel == 2 ? mw[u][2] : mw[u][3];
      const int rank = __popcll(mine & below) + (wsel > 0 ? __popcll(mw[u][0]) : 0) +
                       (wsel > 1 ? __popcll(mw[u][1]) : 0) + (wsel > 2 ? __popcll(mw[u][2]) : 0);
      const int pos = base[u] + rank;
      const int64_t f = (int64_t)t * k + r0 + u;
      row_token[pos] = t;
      row_w[pos] = wv[u];
      slot_row[f] = pos;
    }
  }
}

}  // namespace lmoe
