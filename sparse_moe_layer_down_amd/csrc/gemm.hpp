// MFMA GEMM for gfx950: C[M, N] = A[M, K] . B[N, K]^T with fp32 accumulation.
//
// One template covers every contraction of the layer:
//   dense   W_down, router (sigmoid epilogue), shared experts, W_up
//   grouped routed experts: a device-side tile table maps each M tile to one
//           expert's run of dispatched rows, so no host synchronisation is
//           needed to learn the per-expert row counts
// Fused epilogues:
//   EPI_STORE     C = acc                                  (work dtype or fp32)
//   EPI_SIGMOID   C = sigmoid(acc + col_bias[col])         (router scores, fp32)
//   EPI_GLU       C = SiTU(acc_W1; beta1) * softcap(acc_W2; beta2)
//                 ("Kimi K3 Architecture Deep Dive" §1, SiTU-GLU): the B tile
//                 interleaves 32-row blocks of W1 and W2 for the same hidden
//                 units so both products of one hidden unit land in the same
//                 lane and register
//   EPI_ROWSCALE  C[row] = row_scale[row] * acc            (routing weight g)
//
// Tiling: BM x BN output tile per work-group of WM x WN waves; BK = 128 bytes
// of K per step (64 bf16 or 32 fp32).  Operands go global -> registers -> LDS,
// double buffered; LDS rows are 128 B with the 16-B chunks XOR-swizzled by
// (row & 7) so the MFMA fragment reads of 32 rows at one K offset spread
// over all banks.  bf16 uses v_mfma_f32_32x32x16_bf16 (each lane holds 8
// consecutive K of one row); fp32 uses v_mfma_f32_32x32x2_f32, eight per
// 16-K group with the same per-lane 8-element K slice, so A and B share one
// K assignment and the products sum correctly.
#pragma once
#include "common.hpp"

namespace lmoe {

enum { EPI_STORE = 0, EPI_SIGMOID = 1, EPI_GLU = 2, EPI_ROWSCALE = 3 };

struct GemmArgs {
  const void *A;            // [rows, lda]
  int64_t lda;
  const int32_t *a_rows;    // GATHER: source row of A for each dispatched row
  const void *B;            // [N, ldb] (GLU: W1 rows)
  const void *B2;           // GLU: W2 rows
  int64_t ldb;
  int64_t b_group_stride;   // GROUPED: elements between experts' B matrices
  int64_t kb_len;           // B is split along K into batches of kb_len columns,
  int64_t kb_stride;        //   batch s starts at B + s * kb_stride
  void *C;
  int64_t ldc;
  int M, N, K;              // dense M; N = rows of B (GLU: 2 x hidden units)
  const int4 *tiles;        // GROUPED: {expert, row_begin, row_end, 0}
  const int32_t *ntiles;    // GROUPED: number of valid tiles (device)
  int tiles_m, tiles_n;     // dense M tiles (grouped: max tiles) and N tiles
  int n_logical;            // tiles_m * tiles_n
  int xcd_chunk;
  const float *row_scale;   // EPI_ROWSCALE
  const float *col_bias;    // EPI_SIGMOID (may be null)
  float beta1, beta2;
};

template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int CPL = 1;  // 16-B chunks per lane per 16-K group
  static LMOE_DEV void run(const u32x4 *a, const u32x4 *b, f32x16 &c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                 __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int CPL = 2;
  // Bit-cast whole vectors, then index: element-wise bit casts of vector
  // elements are folded to element 0 by this compiler.
  static LMOE_DEV void run(const u32x4 *a, const u32x4 *b, f32x16 &c) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 av = __builtin_bit_cast(f32x4, a[h]);
      const f32x4 bv = __builtin_bit_cast(f32x4, b[h]);
#pragma unroll
      for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[i], c, 0, 0, 0);
    }
  }
};

LMOE_DEV int swz(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <typename T, typename TO, int BM, int BN, int WM, int WN, int EPI, bool GATHER, bool GROUPED>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int BKE = 128 / (int)sizeof(T);
  constexpr int CPL = Mma<T>::CPL;
  constexpr int NG = BKE / 16;
  constexpr int RPP = NT / 8;  // rows covered per load pass (8 threads x 16 B per row)
  constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
  constexpr int EPT = 16 / (int)sizeof(T);  // elements per 16-B chunk
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of the load pass");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(EPI != EPI_GLU || TN % 2 == 0, "GLU needs W1/W2 subtile pairs");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char *const sA0 = smem;
  unsigned char *const sB0 = smem + 2 * BM * 128;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- which tile
  const int lt = xcd_logical_tile(blockIdx.x, p.xcd_chunk);
  if (lt >= p.n_logical) return;
  int64_t m0;
  int rows_valid, nt;
  int64_t b_off = 0;
  if (GROUPED) {
    const int j = lt / p.tiles_n;
    nt = lt % p.tiles_n;
    if (j >= *p.ntiles) return;
    const int4 tl = p.tiles[j];
    m0 = tl.y;
    rows_valid = tl.z - tl.y;
    b_off = (int64_t)tl.x * p.b_group_stride;
  } else {
    constexpr int GM = 8;
    const int span = GM * p.tiles_n;
    const int g = lt / span, first = g * GM;
    const int gsz = min(p.tiles_m - first, GM);
    const int mt = first + (lt % span) % gsz;
    nt = (lt % span) / gsz;
    m0 = (int64_t)mt * BM;
    rows_valid = min(BM, p.M - (int)m0);
  }

  // ---- per-thread source rows
  const int lrow = tid >> 3, lchunk = tid & 7;
  const T *a_src[A_LD];
  bool a_ok[A_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    const int r = lrow + i * RPP;
    a_ok[i] = r < rows_valid;
    int64_t src = m0 + r;
    if (GATHER) src = a_ok[i] ? (int64_t)p.a_rows[m0 + r] : 0;
    else if (!a_ok[i]) src = 0;
    a_src[i] = (const T *)p.A + src * p.lda + lchunk * EPT;
  }
  const T *b_src[B_LD];
  bool b_ok[B_LD];
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int br = lrow + i * RPP;
    int64_t row;
    const T *base;
    if (EPI == EPI_GLU) {
      const int wcol = br / WTN, within = br % WTN, j = within / 32;
      row = (int64_t)nt * (BN / 2) + wcol * (WTN / 2) + (j / 2) * 32 + (br & 31);
      b_ok[i] = row < p.N / 2;
      base = (const T *)((j & 1) ? p.B2 : p.B);
    } else {
      row = (int64_t)nt * BN + br;
      b_ok[i] = row < p.N;
      base = (const T *)p.B;
    }
    if (!b_ok[i]) row = 0;
    b_src[i] = base + b_off + row * p.ldb + lchunk * EPT;
  }

  const int nk = p.K / BKE;
  u32x4 ra[A_LD], rb[B_LD];
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto gload = [&](int kt) {
    const int64_t k0 = (int64_t)kt * BKE;
    const int64_t s = k0 / p.kb_len;
    const int64_t boff = s * p.kb_stride + (k0 - s * p.kb_len);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = a_ok[i] ? *(const u32x4 *)(a_src[i] + k0) : zero;
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = b_ok[i] ? *(const u32x4 *)(b_src[i] + boff) : zero;
  };
  auto lstore = [&](int buf) {
    unsigned char *sA = sA0 + buf * BM * 128;
    unsigned char *sB = sB0 + buf * BN * 128;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(u32x4 *)(sA + swz(lrow + i * RPP, lchunk)) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *(u32x4 *)(sB + swz(lrow + i * RPP, lchunk)) = rb[i];
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  // wave-uniform: which M subtiles hold valid rows
  bool tm_on[TM];
#pragma unroll
  for (int a = 0; a < TM; ++a) tm_on[a] = (wm * WTM + a * 32) < rows_valid;

  gload(0);
  lstore(0);
  __syncthreads();

  const int half = lane >> 5, l32 = lane & 31;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const unsigned char *sA = sA0 + buf * BM * 128;
    const unsigned char *sB = sB0 + buf * BN * 128;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      u32x4 af[TM][CPL], bfg[TN][CPL];
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int r = wm * WTM + a * 32 + l32;
#pragma unroll
        for (int c = 0; c < CPL; ++c) af[a][c] = *(const u32x4 *)(sA + swz(r, g * 2 * CPL + half * CPL + c));
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int r = wn * WTN + b * 32 + l32;
#pragma unroll
        for (int c = 0; c < CPL; ++c) bfg[b][c] = *(const u32x4 *)(sB + swz(r, g * 2 * CPL + half * CPL + c));
      }
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        if (GROUPED && !tm_on[a]) continue;
#pragma unroll
        for (int b = 0; b < TN; ++b) Mma<T>::run(af[a], bfg[b], acc[a][b]);
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  TO *C = (TO *)p.C;
#pragma unroll
  for (int a = 0; a < TM; ++a) {
    if (!tm_on[a]) continue;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rl = wm * WTM + a * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
      if (rl >= rows_valid) continue;
      const int64_t grow = m0 + rl;
      if (EPI == EPI_GLU) {
#pragma unroll
        for (int b = 0; b < TN; b += 2) {
          const int64_t h = (int64_t)nt * (BN / 2) + wn * (WTN / 2) + (b / 2) * 32 + l32;
          if (h < p.N / 2) {
            const float v = situf_(acc[a][b][i], p.beta1) * softcapf_(acc[a][b + 1][i], p.beta2);
            C[grow * p.ldc + h] = from_f32<TO>(v);
          }
        }
      } else {
        const float rs = (EPI == EPI_ROWSCALE) ? p.row_scale[grow] : 1.0f;
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int64_t col = (int64_t)nt * BN + wn * WTN + b * 32 + l32;
          if (col >= p.N) continue;
          float v = acc[a][b][i];
          if (EPI == EPI_SIGMOID) {
            if (p.col_bias) v += p.col_bias[col];
            v = sigmoidf_(v);
          } else if (EPI == EPI_ROWSCALE) {
            v *= rs;
          }
          C[grow * p.ldc + col] = from_f32<TO>(v);
        }
      }
    }
  }
}

}  // namespace lmoe
