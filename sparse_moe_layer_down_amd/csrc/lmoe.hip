// C ABI of the Stable LatentMoE forward pass and Quantile Balancing (gfx950).
//
// The host code validates every argument, carves the caller's workspace and
// enqueues the kernels on the caller's stream.  It never allocates, never
// synchronises with the device and keeps no state beyond launch settings
// looked up once per kernel and device.
//
// Forward launch sequence ("Kimi K3 Architecture Deep Dive" §1-§3; "Inside
// K3"; LeiPhone report "LatentMoE: paying for a bigger pool" and "Keeping the
// numbers in range"):
//   1 gemm   z = x W_down^T
//   2 gemm   s = sigmoid(z W_r^T + o)                 (fp32 scores)
//   3 topk   biased top-k, routing weights g
//   4 perm   chunk masks -> scan (offsets, tile tables) -> scatter
//   5 gemm   gated hidden of every expert row, one grouped launch: routed
//            experts on their gathered rows, shared experts on all tokens
//            (SiTU-GLU epilogue)
//   6 gemm   W3 of every expert row scaled by g (1 for shared rows) -> one
//            staged row per expert row (fp16, or fp32 when uncapped / fp32)
//   7 norm   u = sum of the token's staged rows; v = RMSNorm(u)
//   8 gemm   y = v W_up^T
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "../../include/lmoe.h"
#include "bwd.hpp"
#include "gemm.hpp"
#include "norm.hpp"
#include "qb.hpp"
#include "route.hpp"

using namespace lmoe;

namespace {

// Tile configurations (BM, BN, waves WM x WN, B prefetch distance PF).  Dense
// GEMMs are MFMA-bound; the grouped expert GEMMs stream the expert bank from
// HBM, with an M tile tall enough to cover a typical expert's rows so each
// expert's weights are read once.
template <int BM_, int BN_, int WM_, int WN_, int PF_, bool BD_ = false> struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, PF = PF_;
  static constexpr bool BD = BD_;  // B straight into LDS (three stages)
};
using CfgDense = Cfg<256, 256, 2, 4, 2, true>;
using CfgRouter = Cfg<128, 256, 2, 4, 2, true>;  // N = n = 896 gives 4 N tiles, 64 x 4 = 256 tiles at T = 8192
using CfgMid = Cfg<128, 128, 2, 2, 1>;     // dense GEMMs whose 256 x 256 tiles would not fill the GPU
using CfgSkinny = Cfg<64, 256, 1, 4, 2>;   // dense GEMMs with M <= 64 (decode), always split-K
using CfgW12 = Cfg<192, 256, 2, 4, 2, true>;
using CfgUp = Cfg<192, 256, 2, 4, 2, true>;      // W_up (N = d): 192-row tiles divide its tile rounds better
using CfgW3 = Cfg<192, 256, 2, 4, 2, true>;
// the backward's expert data-gradient GEMMs read the expert weights in their
// stored [K, N] layout, transposed on the way into LDS (through registers)
using CfgExpertKN = Cfg<192, 256, 2, 4, 1, false>;
// experts with few rows each (decode): 32-row tiles
using CfgW12Small = Cfg<32, 256, 1, 4, 2>;
using CfgW3Small = Cfg<32, 256, 1, 4, 2>;
constexpr int SMALL_ROWS_PER_EXPERT = 24;  // average rows per expert below which the small tiles are used

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t align256(int64_t a) { return (a + 255) & ~(int64_t)255; }

struct WsLayout {
  int64_t off[32];
  int64_t total;
};

enum {
  R_Z = 0, R_COUNTS, R_OFFS, R_ROW_TOKEN, R_SLOT_ROW, R_HIDDEN, R_ROWS, R_V,
  R_SCORES, R_IDX, R_W, R_MASKS, R_CBASE, R_TILES1, R_TILES2, R_NTILES, R_ROW_W, R_PART, R_COUNT_
};

// upper bound of sum_e ceil(count_e / bm) over any routing
// upper bound of the table: routed tiles plus each shared expert's cdiv(T, bm)
int64_t max_tiles(const lmoe_dims &d, int bm) { return d.n + cdiv(d.T * d.k, bm) + d.n_shared * cdiv(d.T, bm); }
// expert rows: T*k routed (dispatch order), then T per shared expert
int64_t expert_rows(const lmoe_dims &d) { return d.T * (d.k + d.n_shared); }

bool small_experts(const lmoe_dims &d) { return d.T * d.k <= SMALL_ROWS_PER_EXPERT * d.n; }
int w12_bm(const lmoe_dims &d) { return small_experts(d) ? CfgW12Small::BM : CfgW12::BM; }
int w3_bm(const lmoe_dims &d) { return small_experts(d) ? CfgW3Small::BM : CfgW3::BM; }

// Split-K plan of a dense GEMM: used when its tiles cannot fill the GPU.
struct SplitPlan {
  int splits, ksteps;
};
template <typename C>
SplitPlan split_plan(int64_t M, int64_t N, int64_t K, int bke, bool force) {
  const int64_t tiles = cdiv(M, C::BM) * cdiv(N, C::BN);
  const int nk = (int)(K / bke);
  if (tiles <= 0 || nk < 4 || (!force && tiles >= 256)) return {1, std::max(nk, 1)};
  int splits = (int)std::min<int64_t>(cdiv(512, tiles), nk / 2);
  splits = std::max(splits, 1);
  int ksteps = (int)cdiv(nk, splits);
  if (ksteps % 2 && nk % 2 == 0) ++ksteps;  // even ranges keep the cross-tile prefetch
  return {(int)cdiv(nk, ksteps), ksteps};
}
// How a dense GEMM is run: M <= 64 -> skinny tile with split-K; otherwise the
// large tile if it yields enough work-groups, else the 128 x 128 tile, split
// along K only if even that leaves the GPU mostly idle.
enum DenseMode { DM_LARGE = 0, DM_MID = 1, DM_MID_SPLIT = 2, DM_SKINNY = 3 };
struct DensePlan {
  DenseMode mode;
  SplitPlan sp;
};
template <typename C>
DensePlan dense_plan(int64_t M, int64_t N, int64_t K, int bke) {
  if (M <= CfgSkinny::BM) return {DM_SKINNY, split_plan<CfgSkinny>(M, N, K, bke, true)};
  if (cdiv(M, C::BM) * cdiv(N, C::BN) >= 256) return {DM_LARGE, {1, (int)(K / bke)}};
  if (cdiv(M, CfgMid::BM) * cdiv(N, CfgMid::BN) >= 128) return {DM_MID, {1, (int)(K / bke)}};
  const SplitPlan sp = split_plan<CfgMid>(M, N, K, bke, true);
  return {sp.splits > 1 ? DM_MID_SPLIT : DM_MID, sp};
}
// fp32 partial-sum bytes a dense GEMM needs (0 when it runs without split-K)
template <typename C>
int64_t part_bytes(int64_t M, int64_t N, int64_t K, int bke) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  const DensePlan pl = dense_plan<C>(M, N, K, bke);
  return (pl.mode == DM_SKINNY || pl.mode == DM_MID_SPLIT) ? (int64_t)pl.sp.splits * M * N * 4 : 0;
}

WsLayout layout(const lmoe_dims &d, int dtype) {
  const int64_t es = dtype == LMOE_BF16 ? 2 : 4;
  const int bke = (int)(128 / es);
  const int64_t nch = cdiv(d.T, PERM_CHUNK);
  int64_t sz[R_COUNT_];
  sz[R_Z] = d.T * d.L * es;
  sz[R_COUNTS] = d.n * 4;
  sz[R_OFFS] = (d.n + 1) * 4;
  sz[R_ROW_TOKEN] = expert_rows(d) * 4;
  sz[R_SLOT_ROW] = d.T * d.k * 4;
  sz[R_HIDDEN] = expert_rows(d) * d.D * es;
  // staged expert outputs, one row per expert row: fp16 (bf16 inputs) or fp32
  sz[R_ROWS] = expert_rows(d) * d.L * 4;  // fp32 rows at most (fp16 when bf16 and both caps finite)
  sz[R_V] = d.T * d.L * es;
  sz[R_SCORES] = d.T * d.n * 4;
  sz[R_IDX] = d.T * d.k * 4;
  sz[R_W] = d.T * d.k * 4;
  sz[R_MASKS] = nch * d.n * 4 * 8;
  sz[R_CBASE] = nch * d.n * 4;
  sz[R_TILES1] = max_tiles(d, w12_bm(d)) * 16;
  sz[R_TILES2] = max_tiles(d, w3_bm(d)) * 16;
  sz[R_NTILES] = (2 + 2 * SCHED_COUNTERS) * 4;  // two table lengths, then each grouped GEMM's tile counters
  sz[R_ROW_W] = expert_rows(d) * 4;
  // split-K partial sums: the dense GEMMs run one after another and share one buffer
  int64_t part = std::max(part_bytes<CfgDense>(d.T, d.L, d.d, bke), part_bytes<CfgRouter>(d.T, d.n, d.L, bke));
  part = std::max(part, part_bytes<CfgUp>(d.T, d.d, d.L, bke));
  sz[R_PART] = part;
  WsLayout w;
  int64_t o = 0;
  for (int i = 0; i < R_COUNT_; ++i) {
    w.off[i] = o;
    o += align256(sz[i]);
  }
  w.total = o;
  return w;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(const lmoe_dims *d) {
  if (!d) return LMOE_ERR_NULL;
  if (d->T < 0 || d->d <= 0 || d->L <= 0 || d->n <= 0 || d->k <= 0 || d->D <= 0 || d->n_shared < 0)
    return LMOE_ERR_SHAPE;
  if (d->L * 2 != d->d) return LMOE_ERR_SHAPE;  // latent is half the model width
  if (d->d % 128 || d->D % 64) return LMOE_ERR_SHAPE;
  if (d->n > 1024 || d->k > d->n || d->k > 64 || d->n_shared > 8) return LMOE_ERR_SHAPE;
  if (d->L > 8192 || d->d > 65536 || d->D > 65536) return LMOE_ERR_SHAPE;
  if (d->T * (d->k + d->n_shared) >= (int64_t)1 << 31) return LMOE_ERR_SHAPE;
  return LMOE_OK;
}

// Compute units of the current device (cached per device).
constexpr int MAX_DEVICES = 64;

// Current device, or -1 if it cannot be used as a cache index.
int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return -1;
  return dev;
}

int device_cus() {
  static std::atomic<int> cus[MAX_DEVICES];  // 0 until queried
  const int dev = current_device();
  if (dev < 0) return 256;
  int v = cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Persistent launch: one work-group per resident slot (CUs x work-groups per
// CU), each walking its share of the logical tiles.
template <typename C, typename T, typename TO, int EPI, bool GATHER, bool GROUPED, bool BKN = false>
hipError_t launch_gemm(GemmArgs a, hipStream_t st) {
  constexpr int threads = 64 * C::WM * C::WN;
  constexpr bool staged = StagedStore<TO, EPI, C::BN / C::WN, C::BN / C::WN / 32>::value;
  // grouped GEMMs: two more ints of LDS publish the next tile taken from the counters
  constexpr bool bd = C::BD;
  constexpr int lds = (bd ? 2 * C::BM * 128 + 3 * C::BN * 128  // staging lives in a B stage
                          : 2 * (C::BM + C::BN) * 128 + (staged ? (threads / 64) * STAGE_BYTES_PER_WAVE : 0)) +
                      (GROUPED ? 16 : 0);
  auto kern = gemm_kernel<T, TO, C::BM, C::BN, C::WM, C::WN, C::PF, EPI, GATHER, GROUPED, bd, BKN>;
  // once per device (and per kernel): raise the kernel's LDS limit and query
  // how many of its work-groups fit on a CU
  struct PerDevice {
    std::once_flag once;
    hipError_t attr = hipSuccess;
    int occ = 1;
  };
  static PerDevice per_dev[MAX_DEVICES];
  const int dev = current_device();
  if (dev < 0) return hipErrorInvalidDevice;
  PerDevice &pd = per_dev[dev];
  std::call_once(pd.once, [&] {
    pd.attr = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    int o = 0;
    if (pd.attr == hipSuccess &&
        (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, threads, lds) != hipSuccess || o <= 0))
      o = 1;
    pd.occ = std::max(o, 1);
  });
  if (pd.attr != hipSuccess) return pd.attr;
  const int occ = pd.occ;
  constexpr int bke = 128 / (int)sizeof(T);
  a.tiles_n = (int)cdiv(a.N, C::BN);
  if (GROUPED && a.krange) {  // every K-range entry covers all M x N tiles of its group
    a.kr_tn = a.tiles_n;
    a.tiles_n *= (int)cdiv(a.M, C::BM);
  }
  if (!GROUPED) a.tiles_m = (int)cdiv(a.M, C::BM);
  a.n_logical = a.tiles_m * a.tiles_n * (GROUPED ? 1 : std::max(a.splits, 1));
  if (a.n_logical == 0) return hipSuccess;
  if constexpr (bd) {
    // the load-to-LDS path addresses A and each B matrix through 32-bit byte
    // offsets (buffer loads): both must span less than 4 GiB; B is one matrix
    // along K (no K batches)
    const int64_t arows = GROUPED && !a.krange ? a.a_nrows : a.M;
    if (arows <= 0 || arows * a.lda * (int64_t)sizeof(T) >= ((int64_t)1 << 32) ||
        (int64_t)a.N * a.ldb * (int64_t)sizeof(T) >= ((int64_t)1 << 32) || (a.kb_len != 0 && a.kb_len != a.K))
      return hipErrorInvalidValue;
  }
  const int nk_all = a.K / bke;
  // cross-tile prefetch needs every tile's step count to be a multiple of 2 (LDS
  // buffer parity) and of the number of register sets
  constexpr int xm = (C::PF % 2 == 0) ? C::PF : 2 * C::PF;
  // (K-range tiles have varying step counts, at least two each by construction
  // of their table; the load-to-LDS pipeline indexes its stages by a global step
  // count, so it prefetches across them)
  a.xpf = a.krange ? (C::BD ? 1 : 0) : (nk_all % xm == 0) && (a.splits <= 1 || a.ksteps % xm == 0);
  int64_t grid = std::min<int64_t>(a.n_logical, (int64_t)device_cus() * occ);
  if (grid >= 8) grid = grid / 8 * 8;
  if (a.kb_len == 0) a.kb_len = a.K;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), lds, st, a);
  return hipGetLastError();
}

// Dense GEMM with the tiling chosen by dense_plan.  Split-K writes fp32
// partials to `part`, then the finalize kernel sums them and applies the
// epilogue.
template <typename C, typename T, typename TO, int EPI>
hipError_t launch_dense(GemmArgs a, float *part, hipStream_t st) {
  constexpr int bke = 128 / (int)sizeof(T);
  const DensePlan pl = dense_plan<C>(a.M, a.N, a.K, bke);
  if (pl.mode == DM_LARGE) return launch_gemm<C, T, TO, EPI, false, false>(a, st);
  if (pl.mode == DM_MID) return launch_gemm<CfgMid, T, TO, EPI, false, false>(a, st);
  GemmArgs b = a;
  b.C = part;
  b.ldc = a.N;
  b.splits = pl.sp.splits;
  b.ksteps = pl.sp.ksteps;
  b.b_split_row = is_glu<EPI> ? a.N / 2 : a.N;
  if (!is_glu<EPI>) b.B2 = nullptr;
  hipError_t e = (pl.mode == DM_SKINNY) ? launch_gemm<CfgSkinny, T, float, EPI_PARTIAL, false, false>(b, st)
                                        : launch_gemm<CfgMid, T, float, EPI_PARTIAL, false, false>(b, st);
  if (e != hipSuccess) return e;
  const int64_t outs = (int64_t)a.M * (is_glu<EPI> ? a.N / 2 : a.N);
  const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(outs, 256), 8192);
  hipLaunchKernelGGL((splitk_finalize_kernel<TO, EPI>), dim3(blocks), dim3(256), 0, st, part, pl.sp.splits, a.M,
                     a.N, (TO *)a.C, a.ldc, a.col_bias, a.beta1, a.beta2);
  return hipGetLastError();
}

template <typename X> struct TypeTag { using type = X; };

GemmArgs gargs() {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.beta1 = 4.0f;
  a.beta2 = 25.0f;
  a.splits = 1;
  return a;
}

template <typename T>
hipError_t run_forward(const lmoe_dims &d, const lmoe_weights &w, const T *x, T *y, int32_t *topk_idx,
                       float *topk_w, float *scores, unsigned char *ws, hipStream_t st,
                       void *const *ev = nullptr) {
  const WsLayout Lw = layout(d, sizeof(T) == 2 ? LMOE_BF16 : LMOE_F32);
  T *z = (T *)(ws + Lw.off[R_Z]);
  int32_t *counts = (int32_t *)(ws + Lw.off[R_COUNTS]);
  int32_t *offs = (int32_t *)(ws + Lw.off[R_OFFS]);
  int32_t *row_token = (int32_t *)(ws + Lw.off[R_ROW_TOKEN]);
  int32_t *slot_row = (int32_t *)(ws + Lw.off[R_SLOT_ROW]);
  T *hid = (T *)(ws + Lw.off[R_HIDDEN]);
  T *v = (T *)(ws + Lw.off[R_V]);
  float *s = scores ? scores : (float *)(ws + Lw.off[R_SCORES]);
  int32_t *idx = topk_idx ? topk_idx : (int32_t *)(ws + Lw.off[R_IDX]);
  float *gw = topk_w ? topk_w : (float *)(ws + Lw.off[R_W]);
  uint64_t *masks = (uint64_t *)(ws + Lw.off[R_MASKS]);
  int32_t *cbase = (int32_t *)(ws + Lw.off[R_CBASE]);
  int4 *tiles1 = (int4 *)(ws + Lw.off[R_TILES1]);
  int4 *tiles2 = (int4 *)(ws + Lw.off[R_TILES2]);
  int32_t *ntiles = (int32_t *)(ws + Lw.off[R_NTILES]);
  float *row_w = (float *)(ws + Lw.off[R_ROW_W]);
  // staged expert outputs, one row per expert row: fp16 for bf16 inputs
  // (11-bit mantissa, summed in fp32 by the combine) while both caps are
  // finite, since the gated hidden is then bounded by beta1 * beta2; fp32 for
  // fp32 inputs and for the uncapped ablation (either cap +inf), whose hidden
  // has no bound.  The region is sized for fp32 rows either way.
  unsigned char *ystage = ws + Lw.off[R_ROWS];
  const bool wide_stage = std::isinf(w.beta1) || std::isinf(w.beta2);
  float *part = (float *)(ws + Lw.off[R_PART]);
  const int T_ = (int)d.T, n = (int)d.n, k = (int)d.k, L = (int)d.L, D = (int)d.D, ns = (int)d.n_shared;
  hipError_t e;
#define LMOE_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)
#define LMOE_MARK(i) do { if (ev && ev[i]) LMOE_TRY(hipEventRecord((hipEvent_t)ev[i], st)); } while (0)

  // 1 z = x W_down^T
  LMOE_MARK(0);
  {
    GemmArgs a = gargs();
    a.A = x; a.lda = d.d; a.B = w.w_down; a.ldb = d.d; a.C = z; a.ldc = L;
    a.M = T_; a.N = L; a.K = (int)d.d;
    LMOE_TRY((launch_dense<CfgDense, T, T, EPI_STORE>(a, part, st)));
  }
  if (w.norm == LMOE_NORM_BOTH) {  // the ablation: z normed in place before routing
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(d.T, 4), 65536);
    hipLaunchKernelGGL(rmsnorm_rows_kernel<T>, dim3(blocks), dim3(256), 0, st, z, T_, L, w.rms_eps);
    LMOE_TRY(hipGetLastError());
  }
  // 2 s = sigmoid(z W_r^T + o)
  LMOE_MARK(1);
  {
    GemmArgs a = gargs();
    a.A = z; a.lda = L; a.B = w.w_router; a.ldb = L; a.C = s; a.ldc = n;
    a.M = T_; a.N = n; a.K = L; a.col_bias = w.router_logit_offset;
    LMOE_TRY((launch_dense<CfgRouter, T, float, EPI_SIGMOID>(a, part, st)));
  }
  // 3 top-k + routing weights
  LMOE_MARK(2);
  {
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(d.T, 4), 65536);
    if (n <= 64) hipLaunchKernelGGL(topk_kernel<1>, dim3(blocks), dim3(256), 0, st, s, w.router_bias, T_, n, k, idx, gw);
    else if (n <= 128) hipLaunchKernelGGL(topk_kernel<2>, dim3(blocks), dim3(256), 0, st, s, w.router_bias, T_, n, k, idx, gw);
    else if (n <= 256) hipLaunchKernelGGL(topk_kernel<4>, dim3(blocks), dim3(256), 0, st, s, w.router_bias, T_, n, k, idx, gw);
    else if (n <= 512) hipLaunchKernelGGL(topk_kernel<8>, dim3(blocks), dim3(256), 0, st, s, w.router_bias, T_, n, k, idx, gw);
    else if (n <= 896) hipLaunchKernelGGL(topk_kernel<14>, dim3(blocks), dim3(256), 0, st, s, w.router_bias, T_, n, k, idx, gw);
    else hipLaunchKernelGGL(topk_kernel<16>, dim3(blocks), dim3(256), 0, st, s, w.router_bias, T_, n, k, idx, gw);
    LMOE_TRY(hipGetLastError());
  }
  // 4 permutation (+ the shared experts' rows and tiles)
  LMOE_MARK(3);
  {
    const int nch = (int)cdiv(d.T, PERM_CHUNK);
    hipLaunchKernelGGL(perm_mask_kernel, dim3(nch), dim3(PERM_CHUNK), (size_t)n * 32, st, idx, T_, n, k, masks, cbase);
    LMOE_TRY(hipGetLastError());
    hipLaunchKernelGGL(perm_scan_kernel, dim3(1), dim3(1024), 0, st, cbase, nch, n, T_, k, ns, counts, offs, w12_bm(d),
                       tiles1, w3_bm(d), tiles2, ntiles);
    LMOE_TRY(hipGetLastError());
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nch, (unsigned)cdiv(k, 4)), dim3(PERM_CHUNK), 0, st, idx, gw, T_, n, k,
                       ns, masks, cbase, offs,
                       row_token, row_w, slot_row);
    LMOE_TRY(hipGetLastError());
  }
  // 5 gated hidden of every expert row: routed experts on their dispatched rows,
  // shared experts (ids n ..) on all tokens, one grouped launch
  LMOE_MARK(4);
  {
    GemmArgs a = gargs();
    a.A = z; a.lda = L; a.a_rows = row_token; a.a_nrows = T_; a.B = w.w1; a.B2 = w.w2; a.ldb = L;
    a.Bsh = w.ws1; a.B2sh = w.ws2; a.n_routed = n;
    a.b_group_stride = (int64_t)D * L; a.C = hid; a.ldc = D;
    a.N = 2 * D; a.K = L; a.tiles = tiles1; a.ntiles = ntiles; a.tiles_m = (int)max_tiles(d, w12_bm(d));
    a.sched = ntiles + 2;
    a.beta1 = w.beta1; a.beta2 = w.beta2;
    if (w.gate == LMOE_GATE_CLIP) {
      if (small_experts(d)) LMOE_TRY((launch_gemm<CfgW12Small, T, T, EPI_GLU_CLIP, true, true>(a, st)));
      else LMOE_TRY((launch_gemm<CfgW12, T, T, EPI_GLU_CLIP, true, true>(a, st)));
    } else {
      if (small_experts(d)) LMOE_TRY((launch_gemm<CfgW12Small, T, T, EPI_GLU, true, true>(a, st)));
      else LMOE_TRY((launch_gemm<CfgW12, T, T, EPI_GLU, true, true>(a, st)));
    }
  }
  // 6 + 7: W3 into the staged rows, then the combine reading them, for one
  // staging type
  auto w3_combine = [&](auto tag) -> hipError_t {
    using TS = typename decltype(tag)::type;
    // 6 W3 of every expert row, scaled by its weight (g, or 1 for shared rows)
    LMOE_MARK(5);
    {
      GemmArgs a = gargs();
      a.A = hid; a.lda = D; a.a_nrows = expert_rows(d); a.B = w.w3; a.Bsh = w.ws3; a.n_routed = n; a.ldb = D;
      a.b_group_stride = (int64_t)L * D;
      a.C = (TS *)ystage; a.ldc = L; a.N = L; a.K = D; a.tiles = tiles2; a.ntiles = ntiles + 1;
      a.tiles_m = (int)max_tiles(d, w3_bm(d)); a.row_scale = row_w;
      a.sched = ntiles + 2 + SCHED_COUNTERS;
      if (small_experts(d)) LMOE_TRY((launch_gemm<CfgW3Small, T, TS, EPI_ROWSCALE, false, true>(a, st)));
      else LMOE_TRY((launch_gemm<CfgW3, T, TS, EPI_ROWSCALE, false, true>(a, st)));
    }
    // 7 combine + RMSNorm
    LMOE_MARK(6);
    {
      const int nch8 = L / 8;
      const T *gain = (const T *)w.rms_gain;
      const int no_norm = w.norm == LMOE_NORM_NONE;
      const dim3 wg((unsigned)cdiv(d.T, 4));
      if (nch8 <= 64) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, TS, 1>), wg, dim3(256), 0, st, (const TS *)ystage, slot_row, gain, v, T_, L, k, ns, w.rms_eps, no_norm);
      else if (nch8 <= 128) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, TS, 2>), wg, dim3(256), 0, st, (const TS *)ystage, slot_row, gain, v, T_, L, k, ns, w.rms_eps, no_norm);
      else if (nch8 <= 256) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, TS, 4>), wg, dim3(256), 0, st, (const TS *)ystage, slot_row, gain, v, T_, L, k, ns, w.rms_eps, no_norm);
      else if (nch8 <= 448) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, TS, 7>), wg, dim3(256), 0, st, (const TS *)ystage, slot_row, gain, v, T_, L, k, ns, w.rms_eps, no_norm);
      else if (nch8 <= 512) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, TS, 8>), wg, dim3(256), 0, st, (const TS *)ystage, slot_row, gain, v, T_, L, k, ns, w.rms_eps, no_norm);
      else hipLaunchKernelGGL((combine_rmsnorm_kernel<T, TS, 4>), dim3(T_), dim3(256), 0, st, (const TS *)ystage, slot_row, gain, v, T_, L, k, ns, w.rms_eps, no_norm);
      LMOE_TRY(hipGetLastError());
    }
    return hipSuccess;
  };
  if constexpr (sizeof(T) == 2) {
    if (wide_stage) LMOE_TRY(w3_combine(TypeTag<float>{}));
    else LMOE_TRY(w3_combine(TypeTag<f16>{}));
  } else {
    LMOE_TRY(w3_combine(TypeTag<float>{}));
  }
  // 8 y = v W_up^T
  LMOE_MARK(7);
  {
    GemmArgs a = gargs();
    a.A = v; a.lda = L; a.B = w.w_up; a.ldb = L; a.C = y; a.ldc = d.d;
    a.M = T_; a.N = (int)d.d; a.K = L;
    LMOE_TRY((launch_dense<CfgUp, T, T, EPI_STORE>(a, part, st)));
  }
  LMOE_MARK(8);
#undef LMOE_MARK
#undef LMOE_TRY
  return hipSuccess;
}

// Geometry of the QB histogram launch, a function of (n, nbins) alone so that
// the workspace size is too: experts per work-group, expert groups, and the
// most token runs a launch uses.  Up to 10240 bins a group is a multiple of 4
// experts, as many B-bin LDS histograms as fit in the 160 KB of a CU, at most 32
// (a 128-byte line of a score row), so that each thread reads 16 bytes of a
// score row at once; wider histograms take one expert per group.
// Runs split the tokens so that the launch fills the GPU in one round: as many
// work-groups as are resident at once (one per CU on a 256-CU MI355X when a
// group's histograms take over 80 KB of LDS, two from 64 KB, four when they take
// at most 40 KB, as with 10000 bins and one expert per group).  Each run but a
// lone one stores its counts to a slab of the workspace, and a merge kernel
// sums the slabs.
// Raises a kernel's dynamic LDS limit to `bytes`, once per device and kernel
// (up to 8 kernels).
hipError_t set_lds_limit(const void *kern, int bytes) {
  struct Entry {
    std::atomic<const void *> kern{nullptr};
    std::atomic<int> state{0};  // 0 unset, 1 done, 2 failed
  };
  static Entry table[MAX_DEVICES][8];
  static std::mutex mu;
  const int dev = current_device();
  if (dev < 0) return hipErrorInvalidDevice;
  for (Entry &e : table[dev]) {
    if (e.kern.load(std::memory_order_acquire) == kern) {
      const int st = e.state.load(std::memory_order_acquire);
      if (st != 0) return st == 1 ? hipSuccess : hipErrorInvalidValue;
    }
  }
  std::lock_guard<std::mutex> lock(mu);
  for (Entry &e : table[dev]) {
    const void *k = e.kern.load(std::memory_order_acquire);
    if (k == kern) return e.state.load() == 1 ? hipSuccess : hipErrorInvalidValue;
    if (k == nullptr) {
      const hipError_t r = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      e.state.store(r == hipSuccess ? 1 : 2, std::memory_order_release);
      e.kern.store(kern, std::memory_order_release);
      return r;
    }
  }
  return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);  // table full
}

constexpr int QB_LDS_MAX = 163840;  // LDS of one MI355X CU

struct QbGeom {
  int eg;
  int64_t groups, runs;
};
QbGeom qb_geom(int64_t n, int nbins) {
  QbGeom g;
  const int64_t quads = QB_LDS_MAX / ((int64_t)nbins * 16);  // 4-expert groups that fit in LDS
  g.eg = quads >= 1 ? (int)std::min<int64_t>(std::min<int64_t>(32, 4 * quads), cdiv(n, 4) * 4)
                    : (int)std::max<int64_t>(1, 65536 / ((int64_t)nbins * 4));
  g.groups = cdiv(n, g.eg);
  const int64_t lds = (int64_t)g.eg * nbins * 4;
  const int64_t slots = 256 * std::max<int64_t>(1, std::min<int64_t>(4, QB_LDS_MAX / lds));
  g.runs = std::max<int64_t>(1, std::min<int64_t>(QB_MAX_RUNS, slots / g.groups));
  return g;
}

int64_t qb_part_bytes(int64_t n, int nbins) {
  const QbGeom g = qb_geom(n, nbins);
  return g.runs > 1 ? align256(g.runs * n * nbins * 4) : 0;
}

// The histogram launch of both QB forms: B-bin histograms of every expert over
// the T > 0 tokens, written to hist (accumulate == 0) or added to it.  part:
// the slabs (qb_part_bytes).  MARGIN: the binned value is the margin of the
// score against the token's threshold (bias [n], thr [T]).  pooled (may be
// null): when the launch merges several runs' slabs, it also leaves the pooled
// histogram sum_e hist[e] there and sets *pooled_done.
template <bool MARGIN>
hipError_t launch_qb_hist(const float *scores, int64_t T, int ni, int kb, int32_t *hist, int32_t *part,
                          int accumulate, const float *bias, const float2 *thr, hipStream_t st,
                          unsigned long long *pooled = nullptr, bool *pooled_done = nullptr) {
  const int64_t n = ni;
  const QbGeom g = qb_geom(n, kb);
  // runs of at least 256 tokens
  int64_t runs = std::max<int64_t>(1, std::min<int64_t>(g.runs, cdiv(T, 256)));
  const int64_t tpb = cdiv(T, runs);
  runs = cdiv(T, tpb);
  const int64_t items = g.groups * runs;
  // (the fused merge's grid has one row per QB_MP_SLICE experts, at most 65535)
  const bool fuse_pool = pooled != nullptr && runs > 1 && cdiv(n, QB_MP_SLICE) <= 65535;
  if (pooled_done) *pooled_done = fuse_pool;
  const bool quad = (n % 4) == 0 && (g.eg % 4) == 0;  // every group's width and first expert too
  auto kern = quad ? qb_hist_kernel<MARGIN, true> : qb_hist_kernel<MARGIN, false>;
  const size_t lds = (size_t)g.eg * kb * 4;
  if (lds > 65536 && set_lds_limit((const void *)kern, QB_LDS_MAX) != hipSuccess) return hipErrorInvalidValue;
  // 16-bit slabs when a run's counts fit and each group's counts start 16-byte aligned
  const bool slab16 = runs > 1 && tpb < 65536 && g.eg % 8 == 0 && (n * kb) % 8 == 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)(8 * cdiv(items, 8))), dim3(QB_HIST_THREADS), lds, st, scores,
                     T, ni, kb, g.eg, (int)g.groups, (int)runs, tpb, hist, part, accumulate, bias, thr,
                     fuse_pool ? pooled : nullptr, slab16 ? 1 : 0);
  const uint16_t *part16 = (const uint16_t *)part;
  if (fuse_pool) {
    const dim3 grid((unsigned)cdiv(kb, 64), (unsigned)cdiv(n, QB_MP_SLICE));
    if (slab16)
      hipLaunchKernelGGL(qb_merge_pool_kernel<uint16_t>, grid, dim3(256), 0, st, part16, (int)runs, ni, kb, hist,
                         accumulate, pooled);
    else
      hipLaunchKernelGGL(qb_merge_pool_kernel<int32_t>, grid, dim3(256), 0, st, part, (int)runs, ni, kb, hist,
                         accumulate, pooled);
  } else if (runs > 1) {
    const int64_t cnt = n * kb;
    if (slab16)
      hipLaunchKernelGGL(qb_merge_kernel<uint16_t>, dim3((unsigned)cdiv(cnt, 256)), dim3(256), 0, st, part16,
                         (int)runs, cnt, hist, accumulate);
    else
      hipLaunchKernelGGL(qb_merge_kernel<int32_t>, dim3((unsigned)cdiv(cnt, 256)), dim3(256), 0, st, part,
                         (int)runs, cnt, hist, accumulate);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Backward pass.  Products run in the forward's C = A B^T MFMA GEMM; the expert
// data-gradient products read the expert weights in their stored [K, N] layout
// (transposed on the way into LDS), the other operands whose contraction
// dimension is not contiguous are transposed first (the dense weights and the
// activations, per call):
//   dv = dy W_up;  dW_up = dy^T v                         (dense)
//   norm backward -> du, dg; gain gradient; router backward -> dl
//   da = g (du W3_e)             grouped over expert rows, du rows gathered
//   dp1, dp2 = gate backward     the W1/W2 products recomputed from the stored z
//   dz rows = dp1 W1_e + dp2 W2_e   grouped; + dl W_r; summed per token -> dz
//   dx = dz W_down;  dW_down = dz^T x;  dW_r = dl^T z     (dense)
//   dW1_e = dp1^T z, dW2_e = dp2^T z, dW3_e = (g du)^T a   one K-range GEMM each:
//                                rows gathered and transposed per expert segment
constexpr int BWD_SCHED = 3 * SCHED_COUNTERS;  // tile counters of the three K-range GEMMs

enum {
  B_WUPT = 0, B_WDOWNT, B_WRT, B_DV, B_DU32, B_DU, B_PROD, B_DG, B_DL, B_DA, B_DP, B_DZROWS, B_DZ,
  B_DYT, B_VT, B_DZT, B_XT, B_ZT, B_DLT, B_ZTG, B_DOT, B_DPT, B_AT, B_ENTRIES, B_BLOCKS, B_NB, B_SCHED, B_SCHED2,
  B_PART, B_COLPART, B_COUNT_
};

struct BwdDims {
  int64_t Tp, np, R, kblocks, Kmax;
};
BwdDims bwd_dims(const lmoe_dims &d) {
  BwdDims b;
  b.Tp = cdiv(d.T, 64) * 64;
  b.np = cdiv(d.n, 64) * 64;
  b.R = expert_rows(d);
  // 64-row blocks of the experts' segments (each padded to whole blocks, and to
  // at least two: at most two more blocks per segment), plus one spare block
  b.kblocks = cdiv(b.R, 64) + 2 * (d.n + d.n_shared);
  b.Kmax = (b.kblocks + 1) * 64;
  return b;
}

// The load-to-LDS GEMMs address each operand through 32-bit byte offsets
// (buffer loads), so every matrix they read must span less than 4 GiB; the
// forward's and (backward) the backward's operands, at the work dtype.
bool spans_fit(const lmoe_dims &d, int dtype, bool backward) {
  const int64_t es = dtype == LMOE_BF16 ? 2 : 4;
  int64_t m = std::max({d.T * d.d, d.T * d.L, expert_rows(d) * d.D, d.L * d.d, d.n * d.L, 2 * d.D * d.L});
  if (backward) {
    const BwdDims b = bwd_dims(d);
    m = std::max({m, d.T * b.np, d.d * b.Tp, d.L * b.Tp, b.np * b.Tp, d.L * b.Kmax, 2 * d.D * b.Kmax});
  }
  return m * es < ((int64_t)1 << 32);
}

WsLayout bwd_layout(const lmoe_dims &d, int dtype) {
  const int64_t es = dtype == LMOE_BF16 ? 2 : 4;
  const int bke = (int)(128 / es);
  const BwdDims b = bwd_dims(d);
  const int64_t T = d.T, L = d.L, D = d.D, n = d.n, ns = d.n_shared, k = d.k;
  int64_t sz[B_COUNT_];
  sz[B_WUPT] = L * d.d * es;
  sz[B_WDOWNT] = d.d * L * es;
  sz[B_WRT] = L * b.np * es;
  sz[B_DV] = T * L * 4;
  sz[B_DU32] = T * L * 4;
  sz[B_DU] = T * L * es;
  sz[B_PROD] = T * L * 4;
  sz[B_DG] = T * k * 4;
  sz[B_DL] = T * b.np * es;
  sz[B_DA] = b.R * D * es;
  sz[B_DP] = b.R * 2 * D * es;
  sz[B_DZROWS] = T * (k + ns + 1) * L * es;
  sz[B_DZ] = T * L * es;
  sz[B_DYT] = d.d * b.Tp * es;
  sz[B_VT] = L * b.Tp * es;
  sz[B_DZT] = L * b.Tp * es;
  sz[B_XT] = d.d * b.Tp * es;
  sz[B_ZT] = L * b.Tp * es;
  sz[B_DLT] = b.np * b.Tp * es;
  sz[B_ZTG] = L * b.Kmax * es;
  sz[B_DOT] = L * b.Kmax * es;
  sz[B_DPT] = 2 * D * b.Kmax * es;
  sz[B_AT] = D * b.Kmax * es;
  sz[B_ENTRIES] = (n + ns) * 16;
  sz[B_BLOCKS] = b.kblocks * 16;
  sz[B_NB] = 16;
  sz[B_SCHED] = BWD_SCHED * 4;
  sz[B_SCHED2] = 3 * SCHED_COUNTERS * 4;  // the grouped dgrad / recompute GEMMs
  int64_t part = 0;
  const int64_t dense[6][3] = {{T, L, d.d}, {T, L, b.np}, {T, d.d, L}, {d.d, L, b.Tp}, {L, d.d, b.Tp}, {n, L, b.Tp}};
  for (auto &m : dense) part = std::max(part, part_bytes<CfgDense>(m[0], m[1], m[2], bke));
  sz[B_PART] = part;
  sz[B_COLPART] = (int64_t)COLSUM_SLICES * L * 4;
  WsLayout w;
  int64_t o = 0;
  for (int i = 0; i < B_COUNT_; ++i) {
    w.off[i] = o;
    o += align256(sz[i]);
  }
  w.total = o;
  return w;
}

// out = in^T per batch: in [R, C] (row stride ld_in), out [C, >= cdiv(R, 64) * 64]
template <typename T>
hipError_t launch_transpose(const T *in, int64_t ld_in, int64_t in_bs, T *out, int64_t ld_out, int64_t out_bs, int R,
                            int C, int batches, hipStream_t st, const int4 *blocks = nullptr, int nblk = 0,
                            const int32_t *nb = nullptr, const int32_t *rows = nullptr,
                            const float *rscale = nullptr) {
  const unsigned gy = blocks ? (unsigned)nblk : (unsigned)cdiv(R, 64);
  if (gy == 0 || C == 0 || batches == 0) return hipSuccess;
  constexpr int CT = sizeof(T) == 2 ? 4 : 2;  // column tiles per block (36 KB / 34 KB of LDS)
  hipLaunchKernelGGL((transpose_kernel<T, CT>), dim3((unsigned)cdiv(C, 64 * CT), gy, (unsigned)batches), dim3(256), 0,
                     st, in, ld_in, in_bs, out, ld_out, out_bs, R, C, blocks, nb, rows, rscale);
  return hipGetLastError();
}

template <typename T>
hipError_t run_backward(const lmoe_dims &d, const lmoe_weights &w, const T *x, const T *dy, const int32_t *idx,
                        const float *gw, const float *scores, const unsigned char *fws, const lmoe_grads &g,
                        unsigned char *ws, hipStream_t st) {
  const int dt = sizeof(T) == 2 ? LMOE_BF16 : LMOE_F32;
  const WsLayout F = layout(d, dt);
  const WsLayout B = bwd_layout(d, dt);
  const BwdDims bd = bwd_dims(d);
  const int T_ = (int)d.T, n = (int)d.n, k = (int)d.k, L = (int)d.L, D = (int)d.D, ns = (int)d.n_shared;
  const int dd = (int)d.d, np_ = (int)bd.np, Tp = (int)bd.Tp;
  const int64_t R = bd.R, Kmax = bd.Kmax;
  // the forward's state
  const T *z = (const T *)(fws + F.off[R_Z]);
  const int32_t *counts = (const int32_t *)(fws + F.off[R_COUNTS]);
  const int32_t *offs = (const int32_t *)(fws + F.off[R_OFFS]);
  const int32_t *row_token = (const int32_t *)(fws + F.off[R_ROW_TOKEN]);
  const int32_t *slot_row = (const int32_t *)(fws + F.off[R_SLOT_ROW]);
  const T *hid = (const T *)(fws + F.off[R_HIDDEN]);
  const unsigned char *ystage = fws + F.off[R_ROWS];
  const T *v = (const T *)(fws + F.off[R_V]);
  const int4 *tiles1 = (const int4 *)(fws + F.off[R_TILES1]);
  const int4 *tiles2 = (const int4 *)(fws + F.off[R_TILES2]);
  const int32_t *ntiles = (const int32_t *)(fws + F.off[R_NTILES]);
  const float *row_w = (const float *)(fws + F.off[R_ROW_W]);
  const bool wide_stage = sizeof(T) == 4 || std::isinf(w.beta1) || std::isinf(w.beta2);
  // this call's buffers
  T *wupT = (T *)(ws + B.off[B_WUPT]);
  T *wdownT = (T *)(ws + B.off[B_WDOWNT]);
  T *wrT = (T *)(ws + B.off[B_WRT]);
  float *dv = (float *)(ws + B.off[B_DV]);
  float *du32 = (float *)(ws + B.off[B_DU32]);
  T *du = (T *)(ws + B.off[B_DU]);
  float *prod = (float *)(ws + B.off[B_PROD]);
  float *dg = (float *)(ws + B.off[B_DG]);
  T *dl = (T *)(ws + B.off[B_DL]);
  T *da = (T *)(ws + B.off[B_DA]);
  T *dp = (T *)(ws + B.off[B_DP]);
  T *dzrows = (T *)(ws + B.off[B_DZROWS]);
  T *dz = (T *)(ws + B.off[B_DZ]);
  T *dyT = (T *)(ws + B.off[B_DYT]);
  T *vT = (T *)(ws + B.off[B_VT]);
  T *dzT = (T *)(ws + B.off[B_DZT]);
  T *xT = (T *)(ws + B.off[B_XT]);
  T *zT = (T *)(ws + B.off[B_ZT]);
  T *dlT = (T *)(ws + B.off[B_DLT]);
  T *zTg = (T *)(ws + B.off[B_ZTG]);
  T *doT = (T *)(ws + B.off[B_DOT]);
  T *dpT = (T *)(ws + B.off[B_DPT]);
  T *aT = (T *)(ws + B.off[B_AT]);
  int4 *entries = (int4 *)(ws + B.off[B_ENTRIES]);
  int4 *blocks = (int4 *)(ws + B.off[B_BLOCKS]);
  int32_t *nb = (int32_t *)(ws + B.off[B_NB]);  // [0] block count, [1] entry count
  int32_t *sched = (int32_t *)(ws + B.off[B_SCHED]);
  int32_t *sched2 = (int32_t *)(ws + B.off[B_SCHED2]);
  float *part = (float *)(ws + B.off[B_PART]);
  constexpr int bke = 128 / (int)sizeof(T);
  hipError_t e;
#define LMOE_TRY(x) do { e = (x); if (e != hipSuccess) return e; } while (0)

  // weights transposed (contraction dimension contiguous)
  LMOE_TRY(launch_transpose<T>((const T *)w.w_up, L, 0, wupT, dd, 0, dd, L, 1, st));
  LMOE_TRY(launch_transpose<T>((const T *)w.w_down, dd, 0, wdownT, L, 0, L, dd, 1, st));
  LMOE_TRY(launch_transpose<T>((const T *)w.w_router, L, 0, wrT, np_, 0, n, L, 1, st));
  // dv = dy W_up
  {
    GemmArgs a = gargs();
    a.A = dy; a.lda = dd; a.B = wupT; a.ldb = dd; a.C = dv; a.ldc = L; a.M = T_; a.N = L; a.K = dd;
    LMOE_TRY((launch_dense<CfgDense, T, float, EPI_STORE>(a, part, st)));
  }
  // norm backward, routing-weight gradients; gain gradient
  {
    const T *gain = (const T *)w.rms_gain;
    const int no_norm = w.norm == LMOE_NORM_NONE;
    const dim3 wg((unsigned)cdiv(d.T, 4));
    const int nch8 = L / 8;
    auto go = [&](auto tag) -> hipError_t {
      using TS = typename decltype(tag)::type;
      const TS *ys = (const TS *)ystage;
      if (nch8 <= 64) hipLaunchKernelGGL((norm_bwd_wave_kernel<T, TS, 1>), wg, dim3(256), 0, st, ys, slot_row, gw, gain, dv, du32, du, prod, dg, T_, L, k, ns, w.rms_eps, no_norm);
      else if (nch8 <= 128) hipLaunchKernelGGL((norm_bwd_wave_kernel<T, TS, 2>), wg, dim3(256), 0, st, ys, slot_row, gw, gain, dv, du32, du, prod, dg, T_, L, k, ns, w.rms_eps, no_norm);
      else if (nch8 <= 256) hipLaunchKernelGGL((norm_bwd_wave_kernel<T, TS, 4>), wg, dim3(256), 0, st, ys, slot_row, gw, gain, dv, du32, du, prod, dg, T_, L, k, ns, w.rms_eps, no_norm);
      else if (nch8 <= 448) hipLaunchKernelGGL((norm_bwd_wave_kernel<T, TS, 7>), wg, dim3(256), 0, st, ys, slot_row, gw, gain, dv, du32, du, prod, dg, T_, L, k, ns, w.rms_eps, no_norm);
      else hipLaunchKernelGGL((norm_bwd_wave_kernel<T, TS, 8>), wg, dim3(256), 0, st, ys, slot_row, gw, gain, dv, du32, du, prod, dg, T_, L, k, ns, w.rms_eps, no_norm);
      return hipGetLastError();
    };
    if constexpr (sizeof(T) == 2) {
      if (wide_stage) LMOE_TRY(go(TypeTag<float>{}));
      else LMOE_TRY(go(TypeTag<f16>{}));
    } else {
      LMOE_TRY(go(TypeTag<float>{}));
    }
    if (no_norm) {
      hipLaunchKernelGGL(fill_zero_kernel<T>, dim3((unsigned)cdiv(L, 256)), dim3(256), 0, st, (T *)g.dgamma, (int64_t)L);
    } else {
      float *colpart = (float *)(ws + B.off[B_COLPART]);
      hipLaunchKernelGGL(colsum_partial_kernel, dim3((unsigned)cdiv(L, 256), COLSUM_SLICES), dim3(256), 0, st, prod,
                         T_, L, colpart);
      hipLaunchKernelGGL(colsum_final_kernel<T>, dim3((unsigned)cdiv(L, 256)), dim3(256), 0, st, colpart, L,
                         (T *)g.dgamma);
    }
    LMOE_TRY(hipGetLastError());
  }
  // router backward (dense dl rows, zero off the chosen experts and past n)
  hipLaunchKernelGGL(router_bwd_kernel<T>, dim3((unsigned)cdiv(d.T, 4)), dim3(256), 0, st, scores, idx, gw, dg, T_, n,
                     np_, k, dl);
  LMOE_TRY(hipGetLastError());
  // expert segments for the weight gradients (and tile counters zeroed)
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, st, counts, offs, n, ns, T_, k, bke, entries, blocks, nb,
                     sched, BWD_SCHED + 0);
  LMOE_TRY(hipGetLastError());
  hipLaunchKernelGGL(fill_i32_kernel, dim3(1), dim3(64), 0, st, sched2, (int64_t)3 * SCHED_COUNTERS, 0);
  LMOE_TRY(hipGetLastError());
  // da = g (du W3_e) for every expert row (du rows gathered by token); W3_e [L, D]
  // is read as stored: K = L rows of N = D columns
  {
    GemmArgs a = gargs();
    a.A = du; a.lda = L; a.a_rows = row_token; a.B = w.w3; a.Bsh = w.ws3; a.n_routed = n;
    a.ldb = D; a.b_group_stride = (int64_t)L * D; a.C = da; a.ldc = D; a.N = D; a.K = L; a.tiles = tiles2;
    a.ntiles = ntiles + 1; a.tiles_m = (int)max_tiles(d, w3_bm(d)); a.row_scale = row_w; a.sched = sched2;
    if (small_experts(d)) LMOE_TRY((launch_gemm<CfgW3Small, T, T, EPI_ROWSCALE, true, true, true>(a, st)));
    else LMOE_TRY((launch_gemm<CfgExpertKN, T, T, EPI_ROWSCALE, true, true, true>(a, st)));
  }
  // gate backward: the W1/W2 products recomputed from z, dp1 | dp2 written [R, 2D]
  {
    GemmArgs a = gargs();
    a.A = z; a.lda = L; a.a_rows = row_token; a.a_nrows = T_; a.B = w.w1; a.B2 = w.w2; a.ldb = L;
    a.Bsh = w.ws1; a.B2sh = w.ws2; a.n_routed = n;
    a.b_group_stride = (int64_t)D * L; a.C = dp; a.ldc = 2 * D;
    a.N = 2 * D; a.K = L; a.tiles = tiles1; a.ntiles = ntiles; a.tiles_m = (int)max_tiles(d, w12_bm(d));
    a.sched = sched2 + SCHED_COUNTERS; a.beta1 = w.beta1; a.beta2 = w.beta2; a.aux = da; a.ldaux = D;
    if (w.gate == LMOE_GATE_CLIP) {
      if (small_experts(d)) LMOE_TRY((launch_gemm<CfgW12Small, T, T, EPI_GLU_CLIP_BWD, true, true>(a, st)));
      else LMOE_TRY((launch_gemm<CfgW12, T, T, EPI_GLU_CLIP_BWD, true, true>(a, st)));
    } else {
      if (small_experts(d)) LMOE_TRY((launch_gemm<CfgW12Small, T, T, EPI_GLU_BWD, true, true>(a, st)));
      else LMOE_TRY((launch_gemm<CfgW12, T, T, EPI_GLU_BWD, true, true>(a, st)));
    }
  }
  // dz rows = dp1 W1_e + dp2 W2_e in the work dtype (summed per token in fp32
  // below): W1_e and W2_e [D, L] read as stored, one K = 2D contraction whose
  // rows k >= D come from W2_e
  {
    GemmArgs a = gargs();
    a.A = dp; a.lda = 2 * D; a.B = w.w1; a.B2 = w.w2; a.Bsh = w.ws1; a.B2sh = w.ws2; a.n_routed = n; a.ldb = L;
    a.b_group_stride = (int64_t)D * L; a.kb_len = D;
    a.C = dzrows; a.ldc = L; a.N = L; a.K = 2 * D; a.tiles = tiles1; a.ntiles = ntiles;
    a.tiles_m = (int)max_tiles(d, w12_bm(d)); a.sched = sched2 + 2 * SCHED_COUNTERS;
    if (small_experts(d)) LMOE_TRY((launch_gemm<CfgW12Small, T, T, EPI_STORE, false, true, true>(a, st)));
    else LMOE_TRY((launch_gemm<CfgExpertKN, T, T, EPI_STORE, false, true, true>(a, st)));
  }
  // the router's part, dl W_r, as one more row block of dz rows
  {
    GemmArgs a = gargs();
    a.A = dl; a.lda = np_; a.B = wrT; a.ldb = np_; a.C = dzrows + (int64_t)T_ * (k + ns) * L; a.ldc = L;
    a.M = T_; a.N = L; a.K = np_;
    LMOE_TRY((launch_dense<CfgDense, T, T, EPI_STORE>(a, part, st)));
  }
  // dz = sum of the token's dz rows (routed slots, shared experts, router)
  {
    const int nch8 = L / 8;
    const T *gain = (const T *)w.rms_gain;
    const dim3 wg((unsigned)cdiv(d.T, 4));
    if (nch8 <= 64) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, T, 1>), wg, dim3(256), 0, st, dzrows, slot_row, gain, dz, T_, L, k, ns + 1, 0.0f, 1);
    else if (nch8 <= 128) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, T, 2>), wg, dim3(256), 0, st, dzrows, slot_row, gain, dz, T_, L, k, ns + 1, 0.0f, 1);
    else if (nch8 <= 256) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, T, 4>), wg, dim3(256), 0, st, dzrows, slot_row, gain, dz, T_, L, k, ns + 1, 0.0f, 1);
    else if (nch8 <= 448) hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, T, 7>), wg, dim3(256), 0, st, dzrows, slot_row, gain, dz, T_, L, k, ns + 1, 0.0f, 1);
    else hipLaunchKernelGGL((combine_rmsnorm_wave_kernel<T, T, 8>), wg, dim3(256), 0, st, dzrows, slot_row, gain, dz, T_, L, k, ns + 1, 0.0f, 1);
    LMOE_TRY(hipGetLastError());
  }
  // dx = dz W_down
  {
    GemmArgs a = gargs();
    a.A = dz; a.lda = L; a.B = wdownT; a.ldb = L; a.C = g.dx; a.ldc = dd; a.M = T_; a.N = dd; a.K = L;
    LMOE_TRY((launch_dense<CfgDense, T, T, EPI_STORE>(a, part, st)));
  }
  // dense weight gradients: contraction over tokens (transposed, padded to Tp)
  LMOE_TRY(launch_transpose<T>(dy, dd, 0, dyT, Tp, 0, T_, dd, 1, st));
  LMOE_TRY(launch_transpose<T>(v, L, 0, vT, Tp, 0, T_, L, 1, st));
  LMOE_TRY(launch_transpose<T>(dz, L, 0, dzT, Tp, 0, T_, L, 1, st));
  LMOE_TRY(launch_transpose<T>(x, dd, 0, xT, Tp, 0, T_, dd, 1, st));
  LMOE_TRY(launch_transpose<T>(z, L, 0, zT, Tp, 0, T_, L, 1, st));
  LMOE_TRY(launch_transpose<T>(dl, np_, 0, dlT, Tp, 0, T_, np_, 1, st));
  {
    GemmArgs a = gargs();
    a.A = dyT; a.lda = Tp; a.B = vT; a.ldb = Tp; a.C = g.dw_up; a.ldc = L; a.M = dd; a.N = L; a.K = Tp;
    LMOE_TRY((launch_dense<CfgDense, T, T, EPI_STORE>(a, part, st)));
  }
  {
    GemmArgs a = gargs();
    a.A = dzT; a.lda = Tp; a.B = xT; a.ldb = Tp; a.C = g.dw_down; a.ldc = dd; a.M = L; a.N = dd; a.K = Tp;
    LMOE_TRY((launch_dense<CfgDense, T, T, EPI_STORE>(a, part, st)));
  }
  {
    GemmArgs a = gargs();
    a.A = dlT; a.lda = Tp; a.B = zT; a.ldb = Tp; a.C = g.dw_router; a.ldc = L; a.M = n; a.N = L; a.K = Tp;
    LMOE_TRY((launch_dense<CfgDense, T, T, EPI_STORE>(a, part, st)));
  }
  // expert weight gradients: rows gathered and transposed per expert segment
  const int nblk = (int)bd.kblocks;
  LMOE_TRY(launch_transpose<T>(z, L, 0, zTg, Kmax, 0, 0, L, 1, st, blocks, nblk, nb, row_token));
  LMOE_TRY(launch_transpose<T>(du, L, 0, doT, Kmax, 0, 0, L, 1, st, blocks, nblk, nb, row_token, row_w));
  LMOE_TRY(launch_transpose<T>(hid, D, 0, aT, Kmax, 0, 0, D, 1, st, blocks, nblk, nb));
  LMOE_TRY(launch_transpose<T>(dp, 2 * D, 0, dpT, Kmax, 0, 0, 2 * D, 1, st, blocks, nblk, nb));
  auto kgemm = [&](const T *A, int M, const T *Bm, int N, void *C, void *Csh, int64_t cstride, int32_t *sc) {
    GemmArgs a = gargs();
    a.A = A; a.lda = Kmax; a.B = Bm; a.ldb = Kmax; a.C = C; a.Csh = Csh; a.c_group_stride = cstride; a.ldc = N;
    a.M = M; a.N = N; a.K = (int)Kmax; a.kb_len = Kmax; a.krange = 1; a.tiles = entries; a.ntiles = nb + 1;
    a.tiles_m = n + ns; a.n_routed = n; a.sched = sc;
    // (the 256 x 256 dense tile's LDS stages fill the whole 160 KB, with no room
    // for the grouped walk's tile slot)
    return launch_gemm<CfgW12, T, T, EPI_STORE, false, true>(a, st);
  };
  LMOE_TRY(kgemm(dpT, D, zTg, L, g.dw1, g.dws1, (int64_t)D * L, sched));
  LMOE_TRY(kgemm(dpT + (int64_t)D * Kmax, D, zTg, L, g.dw2, g.dws2, (int64_t)D * L, sched + SCHED_COUNTERS));
  LMOE_TRY(kgemm(doT, L, aT, D, g.dw3, g.dws3, (int64_t)L * D, sched + 2 * SCHED_COUNTERS));
#undef LMOE_TRY
  return hipSuccess;
}

}  // namespace

extern "C" {

size_t lmoe_workspace_size(const lmoe_dims *dims, int dtype) {
  if (check_dims(dims) != LMOE_OK || (dtype != LMOE_F32 && dtype != LMOE_BF16)) return 0;
  if (!spans_fit(*dims, dtype, false)) return 0;
  return (size_t)layout(*dims, dtype).total;
}

int64_t lmoe_workspace_offset(const lmoe_dims *dims, int dtype, int region) {
  if (check_dims(dims) != LMOE_OK || (dtype != LMOE_F32 && dtype != LMOE_BF16)) return -1;
  if (region < LMOE_WS_Z || region > LMOE_WS_V) return -1;
  return layout(*dims, dtype).off[region];
}

static int forward_impl(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, void *y,
                        int32_t *topk_idx, float *topk_w, float *scores, void *workspace, size_t workspace_bytes,
                        void *stream, void *const *events) {
  int rc = check_dims(dims);
  if (rc != LMOE_OK) return rc;
  if (!w) return LMOE_ERR_NULL;
  if (dtype != LMOE_F32 && dtype != LMOE_BF16) return LMOE_ERR_DTYPE;
  if (!spans_fit(*dims, dtype, false)) return LMOE_ERR_SHAPE;
  if (!(w->beta1 > 0.0f) || !(w->beta2 > 0.0f) || !(w->rms_eps >= 0.0f) || w->rms_eps == INFINITY ||
      (w->gate != LMOE_GATE_TANH && w->gate != LMOE_GATE_CLIP) || (w->norm != LMOE_NORM_RMS && w->norm != LMOE_NORM_NONE && w->norm != LMOE_NORM_BOTH))
    return LMOE_ERR_VALUE;
  if (dims->T == 0) return LMOE_OK;
  if (!x || !y || !workspace || !w->w_down || !w->w_router || !w->router_bias || !w->w1 || !w->w2 || !w->w3 ||
      !w->rms_gain || !w->w_up)
    return LMOE_ERR_NULL;
  if (dims->n_shared > 0 && (!w->ws1 || !w->ws2 || !w->ws3)) return LMOE_ERR_NULL;
  if (dims->n_shared == 0 && (w->ws1 || w->ws2 || w->ws3)) return LMOE_ERR_SHAPE;
  const void *ptrs[] = {x, y, workspace, w->w_down, w->w_router, w->router_bias, w->router_logit_offset,
                        w->w1, w->w2, w->w3, w->ws1, w->ws2, w->ws3, w->rms_gain, w->w_up,
                        topk_idx, topk_w, scores};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return LMOE_ERR_ALIGN;
  if (workspace_bytes < (size_t)layout(*dims, dtype).total) return LMOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e;
  if (dtype == LMOE_BF16)
    e = run_forward<bf16>(*dims, *w, (const bf16 *)x, (bf16 *)y, topk_idx, topk_w, scores,
                          (unsigned char *)workspace, st, events);
  else
    e = run_forward<float>(*dims, *w, (const float *)x, (float *)y, topk_idx, topk_w, scores,
                           (unsigned char *)workspace, st, events);
  if (e != hipSuccess) (void)hipGetLastError();  // leave no error behind for the caller's next HIP call
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

int lmoe_forward(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, void *y,
                 int32_t *topk_idx, float *topk_w, float *scores, void *workspace, size_t workspace_bytes,
                 void *stream) {
  return forward_impl(dims, w, dtype, x, y, topk_idx, topk_w, scores, workspace, workspace_bytes, stream,
                      nullptr);
}

int lmoe_forward_timed(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, void *y,
                       int32_t *topk_idx, float *topk_w, float *scores, void *workspace, size_t workspace_bytes,
                       void *const *events, int n_events, void *stream) {
  if (!events) return LMOE_ERR_NULL;
  if (n_events != LMOE_N_STAGES + 1) return LMOE_ERR_VALUE;
  return forward_impl(dims, w, dtype, x, y, topk_idx, topk_w, scores, workspace, workspace_bytes, stream, events);
}

}  // extern "C"

// Scratch of lmoe_forward_static: device memory the library itself holds, one
// copy per device (the array is allocated when the code object is loaded on a
// device and kept until the process ends).  On the host the array's name is
// only a stand-in: its device address is looked up once per device and only
// that address is passed to kernels.
static __device__ __align__(256) unsigned char scratch[LMOE_STATIC_SCRATCH_BYTES];

namespace {

struct ScratchAddr {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void *ptr = nullptr;
};

// Device address of the current device's scratch (looked up on the first call
// on that device, with it current), or nullptr with *err set.
void *static_scratch(hipError_t *err) {
  static ScratchAddr addr[MAX_DEVICES];
  const int dev = current_device();
  if (dev < 0) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchAddr &a = addr[dev];
  std::call_once(a.once, [&] { a.err = hipGetSymbolAddress(&a.ptr, HIP_SYMBOL(scratch)); });
  *err = a.err;
  return a.err == hipSuccess ? a.ptr : nullptr;
}

}  // namespace

extern "C" {

int lmoe_forward_static(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, void *y,
                        int32_t *topk_idx, float *topk_w, float *scores, void *stream) {
  int rc = check_dims(dims);
  if (rc != LMOE_OK) return rc;
  if (dtype != LMOE_F32 && dtype != LMOE_BF16) return LMOE_ERR_DTYPE;
  if (!spans_fit(*dims, dtype, false)) return LMOE_ERR_SHAPE;
  const int64_t need = layout(*dims, dtype).total;
  if (need > (int64_t)LMOE_STATIC_SCRATCH_BYTES) return LMOE_ERR_SCRATCH;
  if (dims->T == 0) return forward_impl(dims, w, dtype, x, y, topk_idx, topk_w, scores, nullptr, 0, stream, nullptr);
  hipError_t e;
  void *ws = static_scratch(&e);
  if (!ws) return LMOE_ERR_HIP;
  return forward_impl(dims, w, dtype, x, y, topk_idx, topk_w, scores, ws, LMOE_STATIC_SCRATCH_BYTES, stream, nullptr);
}

// QB update workspace: the pooled histogram (nbins int64), tau (one double), the
// wide solve's completion counter (in an 8-byte slot) and its q of every expert
// (n doubles), then the runs' slabs.
int64_t qb_pooled_bytes(int64_t n, int nbins) { return align256(((int64_t)nbins + QB_POOLED_EXTRA + n) * 8); }

size_t lmoe_qb_workspace_size(int64_t n, int32_t nbins) {
  if (nbins < 1 || nbins > 16384 || n < 1 || n > ((int64_t)1 << 20)) return 0;
  return (size_t)(qb_pooled_bytes(n, nbins) + qb_part_bytes(n, nbins));
}

int lmoe_qb_update(const float *scores, int64_t T, int64_t n, int64_t k, int32_t nbins, int32_t *hist,
                   int accumulate, float *bias, int solve, void *workspace, size_t workspace_bytes,
                   void *stream) {
  if (T < 0 || T >= ((int64_t)1 << 31) || n < 1 || n > ((int64_t)1 << 20) || k < 1 || k > n) return LMOE_ERR_SHAPE;
  if (nbins < 1 || nbins > 16384) return LMOE_ERR_VALUE;
  const bool need_ws = solve || T > 0;
  if (!hist || (T > 0 && !scores) || (solve && !bias) || (need_ws && !workspace)) return LMOE_ERR_NULL;
  if (!aligned16(hist) || (scores && !aligned16(scores)) || (bias && !aligned16(bias)) ||
      (workspace && !aligned16(workspace)))
    return LMOE_ERR_ALIGN;
  if (n * nbins >= ((int64_t)1 << 40)) return LMOE_ERR_SHAPE;
  if (need_ws && workspace_bytes < lmoe_qb_workspace_size(n, nbins)) return LMOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int ni = (int)n, kb = nbins;
  unsigned long long *pooled = solve ? (unsigned long long *)workspace : nullptr;
  bool pooled_done = false;
  if (T > 0) {
    int32_t *part = (int32_t *)((unsigned char *)workspace + qb_pooled_bytes(n, nbins));
    if (launch_qb_hist<false>(scores, T, ni, kb, hist, part, accumulate, nullptr, nullptr, st, pooled,
                              &pooled_done) != hipSuccess)
      return LMOE_ERR_HIP;
  } else if (!accumulate) {
    const int64_t cnt = n * nbins;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)std::min<int64_t>(cdiv(cnt, 256), 4096)), dim3(256), 0, st,
                       hist, cnt, 0);
    if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
  }
  if (solve) {
    if (!pooled_done) {
      hipLaunchKernelGGL(fill_u64_kernel, dim3((unsigned)cdiv(nbins + QB_POOLED_EXTRA, 256)), dim3(256), 0, st, pooled,
                         (int64_t)nbins + QB_POOLED_EXTRA);
      if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
      hipLaunchKernelGGL(qb_pool_kernel, dim3((unsigned)cdiv(nbins, 64), (unsigned)cdiv(n, QB_POOL_SLICE)), dim3(256),
                         0, st, hist, ni, kb, pooled);
      if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
    }
    if (nbins <= 64 * QB_LANE_BINS) {
      hipLaunchKernelGGL(qb_solve_kernel, dim3((unsigned)cdiv(n, QB_SOLVE_EXPERTS)), dim3(64 * (QB_SOLVE_EXPERTS + 1)), 0,
                         st, hist, pooled, ni, kb, (int)k, bias);
    } else {
      double *tau = (double *)(pooled + nbins);
      unsigned int *done = (unsigned int *)(pooled + nbins + 1);
      double *qv = (double *)(pooled + nbins + QB_POOLED_EXTRA);
      // wpb expert regions of nbins int32, or the pooled histogram (nbins int64),
      // then the work-group's completion flag
      const int wpb = (int)std::max<int64_t>(1, std::min<int64_t>(4, (QB_LDS_MAX - 1024) / ((int64_t)nbins * 4)));
      const int flag_off = std::max(wpb * nbins * 4, nbins * 8);
      const int solve_lds = flag_off + 16;
      if (solve_lds > 65536 && set_lds_limit((const void *)qb_solve_wide_kernel, QB_LDS_MAX) != hipSuccess)
        return LMOE_ERR_HIP;
      hipLaunchKernelGGL(qb_solve_wide_kernel, dim3((unsigned)(cdiv(n, wpb) + 1)), dim3(64 * wpb), (size_t)solve_lds, st,
                         hist, pooled, tau, done, qv, ni, kb, (int)k, wpb, flag_off, bias);
    }
    if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
  }
  return LMOE_OK;
}

size_t lmoe_backward_workspace_size(const lmoe_dims *dims, int dtype) {
  if (check_dims(dims) != LMOE_OK || (dtype != LMOE_F32 && dtype != LMOE_BF16) || dims->L > 4096) return 0;
  if (!spans_fit(*dims, dtype, true)) return 0;
  return (size_t)bwd_layout(*dims, dtype).total;
}

int lmoe_backward(const lmoe_dims *dims, const lmoe_weights *w, int dtype, const void *x, const void *dy,
                  const int32_t *topk_idx, const float *topk_w, const float *scores, const void *fwd_workspace,
                  size_t fwd_workspace_bytes, const lmoe_grads *grads, void *workspace, size_t workspace_bytes,
                  void *stream) {
  int rc = check_dims(dims);
  if (rc != LMOE_OK) return rc;
  if (dims->L > 4096) return LMOE_ERR_SHAPE;
  if (!w || !grads) return LMOE_ERR_NULL;
  if (dtype != LMOE_F32 && dtype != LMOE_BF16) return LMOE_ERR_DTYPE;
  if (!spans_fit(*dims, dtype, true)) return LMOE_ERR_SHAPE;
  if (!(w->beta1 > 0.0f) || !(w->beta2 > 0.0f) || !(w->rms_eps >= 0.0f) || w->rms_eps == INFINITY ||
      (w->gate != LMOE_GATE_TANH && w->gate != LMOE_GATE_CLIP) || (w->norm != LMOE_NORM_RMS && w->norm != LMOE_NORM_NONE))
    return LMOE_ERR_VALUE;
  const lmoe_grads &g = *grads;
  if (!g.dw_down || !g.dw_router || !g.dw1 || !g.dw2 || !g.dw3 || !g.dgamma || !g.dw_up) return LMOE_ERR_NULL;
  if (dims->n_shared > 0 && (!g.dws1 || !g.dws2 || !g.dws3 || !w->ws1 || !w->ws2 || !w->ws3)) return LMOE_ERR_NULL;
  if (dims->n_shared == 0 && (g.dws1 || g.dws2 || g.dws3)) return LMOE_ERR_SHAPE;
  if (dims->T > 0 && (!x || !dy || !g.dx || !topk_idx || !topk_w || !scores || !fwd_workspace || !workspace ||
                      !w->w_down || !w->w_router || !w->w1 || !w->w2 || !w->w3 || !w->rms_gain || !w->w_up))
    return LMOE_ERR_NULL;
  const void *ptrs[] = {x, dy, topk_idx, topk_w, scores, fwd_workspace, workspace, g.dx, g.dw_down, g.dw_router,
                        g.dw1, g.dw2, g.dw3, g.dws1, g.dws2, g.dws3, g.dgamma, g.dw_up, w->w_down, w->w_router,
                        w->w1, w->w2, w->w3, w->ws1, w->ws2, w->ws3, w->rms_gain, w->w_up};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return LMOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const int64_t es = dtype == LMOE_BF16 ? 2 : 4;
  if (dims->T == 0) {  // no tokens: every weight gradient is zero
    const int64_t n = dims->n, ns = dims->n_shared, L = dims->L, D = dims->D, d = dims->d;
    struct { void *p; int64_t cnt; } z[] = {{g.dw_down, L * d}, {g.dw_router, n * L}, {g.dw1, n * D * L},
                                            {g.dw2, n * D * L}, {g.dw3, n * L * D}, {g.dws1, ns * D * L},
                                            {g.dws2, ns * D * L}, {g.dws3, ns * L * D}, {g.dgamma, L}, {g.dw_up, d * L}};
    for (auto &q : z) {
      if (!q.p || q.cnt == 0) continue;
      const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(q.cnt, 256), 65536);
      if (es == 2) hipLaunchKernelGGL(fill_zero_kernel<bf16>, dim3(blocks), dim3(256), 0, st, (bf16 *)q.p, q.cnt);
      else hipLaunchKernelGGL(fill_zero_kernel<float>, dim3(blocks), dim3(256), 0, st, (float *)q.p, q.cnt);
      if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
    }
    return LMOE_OK;
  }
  if (fwd_workspace_bytes < (size_t)layout(*dims, dtype).total) return LMOE_ERR_WORKSPACE;
  if (workspace_bytes < (size_t)bwd_layout(*dims, dtype).total) return LMOE_ERR_WORKSPACE;
  hipError_t e;
  if (dtype == LMOE_BF16)
    e = run_backward<bf16>(*dims, *w, (const bf16 *)x, (const bf16 *)dy, topk_idx, topk_w, scores,
                           (const unsigned char *)fwd_workspace, g, (unsigned char *)workspace, st);
  else
    e = run_backward<float>(*dims, *w, (const float *)x, (const float *)dy, topk_idx, topk_w, scores,
                            (const unsigned char *)fwd_workspace, g, (unsigned char *)workspace, st);
  if (e != hipSuccess) (void)hipGetLastError();
  return e == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

size_t lmoe_qb_margin_workspace_size(int64_t T, int64_t n, int32_t nbins) {
  if (T < 0 || T >= ((int64_t)1 << 31) || nbins < 1 || nbins > 16384 || n < 1 || n > 1024) return 0;
  return (size_t)(align256(std::max<int64_t>(T, 1) * 8) + qb_part_bytes(n, nbins));
}

int lmoe_qb_margin_update(const float *scores, int64_t T, int64_t n, int64_t k, int32_t nbins, int32_t *hist,
                          int accumulate, float *bias, int solve, void *workspace, size_t workspace_bytes,
                          void *stream) {
  if (T < 0 || T >= ((int64_t)1 << 31) || n < 1 || n > 1024 || k < 1 || k > n) return LMOE_ERR_SHAPE;
  if (nbins < 1 || nbins > 16384) return LMOE_ERR_VALUE;
  if (!hist || !bias || (T > 0 && (!scores || !workspace))) return LMOE_ERR_NULL;
  if (!aligned16(hist) || !aligned16(bias) || (scores && !aligned16(scores)) || (workspace && !aligned16(workspace)))
    return LMOE_ERR_ALIGN;
  if (T > 0 && workspace_bytes < lmoe_qb_margin_workspace_size(T, n, nbins)) return LMOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int ni = (int)n, kb = nbins, Ti = (int)T;
  if (T == 0 && !accumulate) {
    const int64_t cnt = n * nbins;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)std::min<int64_t>(cdiv(cnt, 256), 4096)), dim3(256), 0, st,
                       hist, cnt, 0);
    if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
  }
  if (T > 0) {
    float2 *thr = (float2 *)workspace;
    int32_t *part = (int32_t *)((unsigned char *)workspace + align256(T * 8));
    const unsigned blocks = (unsigned)std::min<int64_t>(cdiv(T, 4), 65536);
    if (ni <= 64) hipLaunchKernelGGL(qb_thresholds_kernel<1>, dim3(blocks), dim3(256), 0, st, scores, bias, Ti, ni, (int)k, thr);
    else if (ni <= 128) hipLaunchKernelGGL(qb_thresholds_kernel<2>, dim3(blocks), dim3(256), 0, st, scores, bias, Ti, ni, (int)k, thr);
    else if (ni <= 256) hipLaunchKernelGGL(qb_thresholds_kernel<4>, dim3(blocks), dim3(256), 0, st, scores, bias, Ti, ni, (int)k, thr);
    else if (ni <= 512) hipLaunchKernelGGL(qb_thresholds_kernel<8>, dim3(blocks), dim3(256), 0, st, scores, bias, Ti, ni, (int)k, thr);
    else if (ni <= 896) hipLaunchKernelGGL(qb_thresholds_kernel<14>, dim3(blocks), dim3(256), 0, st, scores, bias, Ti, ni, (int)k, thr);
    else hipLaunchKernelGGL(qb_thresholds_kernel<16>, dim3(blocks), dim3(256), 0, st, scores, bias, Ti, ni, (int)k, thr);
    if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
    if (launch_qb_hist<true>(scores, T, ni, kb, hist, part, accumulate, bias, thr, st) != hipSuccess) return LMOE_ERR_HIP;
  }
  if (solve) {
    hipLaunchKernelGGL(qb_margin_solve_kernel, dim3((unsigned)cdiv(n, 4)), dim3(256), 0, st, hist, ni, kb, (int)k,
                       bias);
    if (hipGetLastError() != hipSuccess) return LMOE_ERR_HIP;
  }
  return LMOE_OK;
}

int lmoe_bias_signsgd(const int32_t *topk_idx, int64_t T, int64_t n, int64_t k, float step, float *bias,
                      void *stream) {
  if (T < 0 || n < 1 || n > ((int64_t)1 << 20) || k < 1 || k > n || T * k >= ((int64_t)1 << 40)) return LMOE_ERR_SHAPE;
  if (!(std::fabs(step) < INFINITY)) return LMOE_ERR_VALUE;
  if (!bias || (T > 0 && !topk_idx)) return LMOE_ERR_NULL;
  if (!aligned16(bias) || (topk_idx && !aligned16(topk_idx))) return LMOE_ERR_ALIGN;
  if (T == 0) return LMOE_OK;  // no loads and a share of zero: every expert is at its share
  hipLaunchKernelGGL(signsgd_kernel, dim3((unsigned)cdiv(n, 256)), dim3(1024), 0, (hipStream_t)stream, topk_idx,
                     T * k, (int)n, step, bias);
  return hipGetLastError() == hipSuccess ? LMOE_OK : LMOE_ERR_HIP;
}

const char *lmoe_strerror(int status) {
  switch (status) {
    case LMOE_OK: return "ok";
    case LMOE_ERR_NULL: return "a required pointer is NULL";
    case LMOE_ERR_SHAPE: return "dimensions violate the layer's or the kernels' rules";
    case LMOE_ERR_DTYPE: return "unknown work dtype";
    case LMOE_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case LMOE_ERR_WORKSPACE: return "workspace smaller than required";
    case LMOE_ERR_HIP: return "a HIP launch or runtime call failed";
    case LMOE_ERR_VALUE: return "a scalar argument is out of range";
    case LMOE_ERR_SCRATCH: return "the call needs more scratch than the library's static buffer holds";
    default: return "unknown status";
  }
}

}  // extern "C"
