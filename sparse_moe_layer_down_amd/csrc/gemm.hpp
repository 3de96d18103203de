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
//   EPI_GLU_CLIP  the same with both caps a hard clip (the cap ablation)
//   EPI_ROWSCALE  C[row] = row_scale[row] * acc            (routing weight g)
//   EPI_PARTIAL   split-K: fp32 partial sums of one K range, C[split][row][col];
//                 a finalize kernel sums the splits and applies the real
//                 epilogue (used when M is too small to fill the GPU).  B rows
//                 from b_split_row on are taken from B2 (W1 and W2 stacked).
//
// Tiling: BM x BN output tile per work-group of WM x WN waves; BK = 128 bytes
// of K per step (64 bf16 or 32 fp32).  Two load pipelines: load to LDS (BDMA,
// below) for the eight-wave tiles, and global -> registers -> LDS for the rest,
// where the global loads run PF steps ahead through a ring of register sets and
// LDS is double buffered.  LDS rows are 128 B with the 16-B chunks XOR-swizzled by
// (row & 7) so the MFMA fragment reads of 32 rows at one K offset spread
// over all banks.  bf16 uses v_mfma_f32_32x32x16_bf16 (each lane holds 8
// consecutive K of one row); fp32 uses v_mfma_f32_32x32x2_f32, eight per
// 16-K group with the same per-lane 8-element K slice, so A and B share one
// K assignment and the products sum correctly.
#pragma once
#include "common.hpp"

namespace lmoe {

enum { EPI_STORE = 0, EPI_SIGMOID = 1, EPI_GLU = 2, EPI_ROWSCALE = 3, EPI_PARTIAL = 4, EPI_GLU_CLIP = 5,
       EPI_GLU_BWD = 6, EPI_GLU_CLIP_BWD = 7 };

// Both gated epilogues: EPI_GLU caps its branches with the tanh softcap,
// EPI_GLU_CLIP with the hard clip clamp(x; beta) = min(max(x, -beta), beta) that
// the softcap replaces at the same ceilings (the cap ablation; "Kimi K3
// Architecture Deep Dive" §1).  The clamp keeps NaN (its comparisons fail).
template <int EPI>
constexpr bool is_glu_bwd = EPI == EPI_GLU_BWD || EPI == EPI_GLU_CLIP_BWD;
// every epilogue that takes W1 and W2 products of the same hidden units
template <int EPI>
constexpr bool is_glu = EPI == EPI_GLU || EPI == EPI_GLU_CLIP || is_glu_bwd<EPI>;

LMOE_DEV float clampf_(float x, float beta) { return x < -beta ? -beta : (x > beta ? beta : x); }

template <int EPI>
LMOE_DEV float glu_(float x1, float x2, float beta1, float beta2) {
  if constexpr (EPI == EPI_GLU_CLIP)
    return clampf_(x1, beta1) * sigmoid_hw(x1) * clampf_(x2, beta2);
  else
    return situf_(x1, beta1) * softcapf_(x2, beta2);
}

// Backward of the gate a = SiTU(x1) C(x2) (C the branch cap): given da,
//   dx1 = da C(x2) SiTU'(x1),  dx2 = da SiTU(x1) C'(x2),
// SiTU'(x) = C'(x) sigmoid(x) + C(x) sigmoid(x) (1 - sigmoid(x)); the softcap's
// C'(x) = 1 - tanh^2(x / beta) = 1 - (C(x) / beta)^2, the clip's 1 inside
// (-beta, beta) and 0 outside.
template <int EPI>
LMOE_DEV void glu_bwd_(float x1, float x2, float da, float beta1, float beta2, float &dx1, float &dx2) {
  const float sg = sigmoid_hw(x1);
  float c1, c2, g1, g2;
  if constexpr (EPI == EPI_GLU_CLIP_BWD) {
    c1 = clampf_(x1, beta1);
    c2 = clampf_(x2, beta2);
    g1 = fabsf(x1) < beta1 ? 1.0f : 0.0f;
    g2 = fabsf(x2) < beta2 ? 1.0f : 0.0f;
  } else {
    c1 = softcapf_(x1, beta1);
    c2 = softcapf_(x2, beta2);
    const float t1 = c1 * (1.0f / beta1), t2 = c2 * (1.0f / beta2);
    g1 = 1.0f - t1 * t1;
    g2 = 1.0f - t2 * t2;
  }
  dx1 = da * c2 * (g1 * sg + c1 * sg * (1.0f - sg));
  dx2 = da * (c1 * sg) * g2;
}

struct GemmArgs {
  const void *A;            // [rows, lda]
  int64_t lda;
  const int32_t *a_rows;    // GATHER: source row of A for each dispatched row
  const void *B;            // [N, ldb] (GLU: W1 rows); BKN: [K, ldb], K rows of N columns
  const void *B2;           // GLU: W2 rows
  int64_t ldb;
  int64_t b_group_stride;   // GROUPED: elements between experts' B matrices
  const void *Bsh;          // GROUPED: the shared experts' bank (expert ids >= n_routed), same stride
  const void *B2sh;         //   and its second matrix (GLU: W2)
  int n_routed;             // GROUPED: expert ids below this index B / B2
  int64_t kb_len;           // B is split along K into batches of kb_len columns,
  int64_t kb_stride;        //   batch s starts at B + s * kb_stride (BKN: K rows >= kb_len
                            //   are rows k - kb_len of B2)
  void *C;
  int64_t ldc;
  int M, N, K;              // dense M; N = rows of B (GLU: 2 x hidden units)
  const int4 *tiles;        // GROUPED: {expert, row_begin, row_end, 0}
  const int32_t *ntiles;    // GROUPED: number of valid tiles (device)
  int tiles_m, tiles_n;     // dense M tiles (grouped: max tiles) and N tiles
  int n_logical;            // tiles_m * tiles_n (dense: x splits)
  int xpf;                  // every tile has an even number of K steps: prefetch across tiles
  const float *row_scale;   // EPI_ROWSCALE
  const float *col_bias;    // EPI_SIGMOID (may be null)
  float beta1, beta2;
  int splits;               // dense split-K: number of K ranges (1 = none)
  int ksteps;               // K steps per range
  int b_split_row;          // EPI_PARTIAL: B rows >= this come from B2
  int32_t *sched;           // GROUPED: 8 tile counters, zero at launch (null: static tile walk)
  const void *aux;          // EPI_GLU_BWD: da [rows, N/2] (work dtype), row stride ldaux
  int64_t ldaux;
  int krange;               // GROUPED K-range mode: table entry e = {group, first K step, K steps, 0};
                            //   every entry covers cdiv(M, BM) x kr_tn tiles of the same A and B
                            //   (rows of A from 0, its K range from the entry), written to
                            //   C + group * c_group_stride (group >= n_routed: Csh + ...)
  int kr_tn;                // K-range: N tiles per entry
  void *Csh;
  int64_t c_group_stride;
  int64_t a_nrows;          // load-to-LDS grouped GEMMs: rows of A (its byte offsets must stay below 4 GiB)
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

// LDS address of 16-B chunk c of tile row r (rows of 128 B).  The chunk is
// XOR-swizzled so that an MFMA fragment read (one chunk column, 32 consecutive
// rows, 16 B per lane) has no bank conflict whether the LDS serves 8 or 16
// lanes per pass: any 8 consecutive rows get 8 distinct chunk slots, and within
// any 16 consecutive rows the even and the odd rows each get 8 distinct slots.
LMOE_DEV int swz(int r, int c) { return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 1)) << 4); }

// The B tile of a GEMM whose B is stored [K, N] (BKN): each thread writes the
// transposed pieces of 8 (bf16) or 4 (fp32) consecutive tile rows, so the chunk
// slot also takes row bits 3..5; fragment reads keep the property above (any 8
// consecutive rows get 8 distinct slots, and within 16 rows the even and the odd
// rows each get 8), and the transposed writes of 8 (16 for 8-byte pieces)
// consecutive lanes fall on distinct banks.
LMOE_DEV int swz_kn(int r, int c) { return r * 128 + ((c ^ (r & 7) ^ ((r >> 3) & 7)) << 4); }

template <int V> struct IC { static constexpr int value = V; };

// One logical tile: rows [m0, m0 + rows) against the B matrices at B / B2
// (grouped: one expert's), N tile nt, split ks covering K steps [kbeg, kbeg + nk).
struct TileI {
  const void *B, *B2;
  void *C;  // output matrix of the tile
  int64_t m0;
  int rows, nt, ks, kbeg, nk;
};

// Logical tile l -> TileI.  Grouped: entry l / tiles_n of the device tile table.
// Dense: split-major, then groups of 8 M tiles walked down before across.
template <typename T, typename TOut, int BM, bool GROUPED>
LMOE_DEV TileI decode_tile(const GemmArgs &p, int l, int nk_all) {
  TileI t;
  t.ks = 0;
  t.B = p.B;
  t.B2 = p.B2;
  t.C = p.C;
  if (GROUPED && p.krange) {
    const int j = l / p.tiles_n, r = l % p.tiles_n;
    const int4 e = p.tiles[j];
    const int mt = r / p.kr_tn;
    t.nt = r % p.kr_tn;
    t.m0 = (int64_t)mt * BM;
    t.rows = min(BM, p.M - (int)t.m0);
    t.kbeg = e.y;
    t.nk = e.z;
    t.C = e.x >= p.n_routed ? (void *)((TOut *)p.Csh + (int64_t)(e.x - p.n_routed) * p.c_group_stride)
                            : (void *)((TOut *)p.C + (int64_t)e.x * p.c_group_stride);
    return t;
  }
  if (GROUPED) {
    const int j = l / p.tiles_n;
    t.nt = l % p.tiles_n;
    const int4 e = p.tiles[j];
    t.m0 = e.y;
    t.rows = e.z - e.y;
    const bool sh = e.x >= p.n_routed;  // a shared expert: rows are all tokens, weights from the shared bank
    const int64_t off = (int64_t)(sh ? e.x - p.n_routed : e.x) * p.b_group_stride;
    const T *b1 = (const T *)(sh ? p.Bsh : p.B), *b2 = (const T *)(sh ? p.B2sh : p.B2);
    t.B = b1 + off;
    t.B2 = b2 ? b2 + off : nullptr;
  } else {
    constexpr int GM = 8;
    const int per_split = p.tiles_m * p.tiles_n;
    t.ks = l / per_split;
    const int lm = l % per_split;
    const int span = GM * p.tiles_n;
    const int g = lm / span, first = g * GM;
    const int gsz = min(p.tiles_m - first, GM);
    const int mt = first + (lm % span) % gsz;
    t.nt = (lm % span) / gsz;
    t.m0 = (int64_t)mt * BM;
    t.rows = min(BM, p.M - (int)t.m0);
  }
  t.kbeg = t.ks * p.ksteps;
  t.nk = (p.splits > 1) ? min(p.ksteps, nk_all - t.kbeg) : nk_all;
  return t;
}

// Epilogue of one output tile.  The MFMA takes the B fragment as its first
// operand, so acc[a][b] is the (B subtile b) x (A subtile a) block: lane l owns
// A row l32 of subtile a (tile row (a * WM + wm) * 32 + l32) and, in registers
// 4g .. 4g+3, the four consecutive B columns 8g + 4 * half .. +3 of subtile b,
// which leave in one vector store.
// Epilogue staging through LDS for 16-bit outputs: each lane's 4-column pieces
// cover only 8 bytes of a line per store, so a wave's slice of 32 rows (64
// output columns, or 32 hidden units for SiTU-GLU) is first written to a
// wave-private 4 KB LDS area (rows of 128 bytes, 16-byte chunks XOR-swizzled by
// row) and read back as whole rows, which leave as 16-byte stores covering full
// lines.
template <typename TO, int EPI, int WTN, int TN>
struct StagedStore {
  static constexpr bool value = (EPI == EPI_ROWSCALE || EPI == EPI_STORE || is_glu<EPI>) &&
                                sizeof(TO) == 2 && WTN == 64 && TN == 2;
};
constexpr int STAGE_BYTES_PER_WAVE = 32 * 128;

template <typename TO, int EPI, int BN, int WTN, int WM, int TM, int TN>
LMOE_DEV void store_tile(const GemmArgs &p, void *Cout, f32x16 (&acc)[TM][TN], int64_t m0, int rows_valid, int nt,
                         int ks, int wm, int wn, int half, int l32, unsigned char *stage) {
  TO *C = (TO *)Cout;
  if constexpr (StagedStore<TO, EPI, WTN, TN>::value) {
    constexpr bool GLU = is_glu<EPI>;
    constexpr bool GBWD = is_glu_bwd<EPI>;  // two outputs per hidden unit: dp1 | dp2
    constexpr int CPR = GLU ? 4 : 8;  // 16-byte chunks of one output per staged row (32 or 64 outputs)
    constexpr int CPRR = GBWD ? 8 : CPR;  // chunks per staged row (gate backward: dp1 in 0..3, dp2 in 4..7)
    const int lane = half * 32 + l32;
    const int nout = GLU ? p.N / 2 : p.N;
    const int64_t c_base = GLU ? (int64_t)nt * (BN / 2) + wn * (WTN / 2) : (int64_t)nt * BN + wn * WTN;
    const bool full = (p.ldc % 8) == 0 && c_base + CPR * 8 <= nout && (!GBWD || (p.ldaux % 4) == 0);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int r0 = (a * WM + wm) * 32;  // first tile row of this subtile
      if (r0 >= rows_valid) continue;     // wave-uniform
      const float rs = (EPI == EPI_ROWSCALE) ? p.row_scale[m0 + min(r0 + l32, rows_valid - 1)] : 1.0f;
      if (full) {
        // the gate backward's da row of this lane (rows past the valid range read a valid row)
        const TO *darow = GBWD ? (const TO *)p.aux + (m0 + min(r0 + l32, rows_valid - 1)) * p.ldaux + c_base + half * 4
                               : nullptr;
        // write: lane (half, l32) owns row l32, outputs (chunk j) * 8 + half*4 .. +3; the
        // 8-byte half also flips with row bit 3, so the 16 lanes of one write pass (rows
        // 0..15 or 16..31, one half) hit 16 distinct 8-byte slots
        const int hoff = (half ^ ((l32 >> 3) & 1)) << 3;
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
          const int b = j / 4, g = j % 4;
          float o[4], o2[4];
          if constexpr (GBWD) {
            const u32x2 dv = *(const u32x2 *)(darow + g * 8);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t w = dv[c >> 1];
              const TO dac = __builtin_bit_cast(TO, (unsigned short)((c & 1) ? (w >> 16) : (w & 0xFFFFu)));
              glu_bwd_<EPI>(acc[a][0][4 * g + c], acc[a][1][4 * g + c], to_f32(dac), p.beta1, p.beta2, o[c], o2[c]);
            }
            store4((TO *)(stage + l32 * 128 + (((j + 4) ^ (l32 & 7)) << 4) + hoff), o2);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if (GLU)
                o[c] = glu_<EPI>(acc[a][0][4 * g + c], acc[a][1][4 * g + c], p.beta1, p.beta2);
              else
                o[c] = acc[a][b][4 * g + c] * rs;
            }
          }
          store4((TO *)(stage + l32 * 128 + ((j ^ (l32 & 7)) << 4) + hoff), o);
        }
        // read back whole rows: CPRR lanes per row (halves swapped back on rows with bit 3 set)
        constexpr int RPI = 64 / CPRR;  // rows per pass
#pragma unroll
        for (int i = 0; i < 32 / RPI; ++i) {
          const int r = lane / CPRR + RPI * i, c = lane % CPRR;
          u32x4 v = *(const u32x4 *)(stage + r * 128 + ((c ^ (r & 7)) << 4));
          if ((r >> 3) & 1) v = u32x4{v[2], v[3], v[0], v[1]};
          if (r0 + r < rows_valid) {
            // gate backward: chunks 4..7 are dp2, H = p.N / 2 columns further on
            const int64_t col = GBWD ? (c < CPR ? c_base + c * 8 : p.N / 2 + c_base + (c - CPR) * 8) : c_base + c * 8;
            u32x4 *dst = (u32x4 *)(C + (m0 + r0 + r) * p.ldc + col);
            // staged expert rows are read once, by the combine: stream them
            if (EPI == EPI_ROWSCALE)
              __builtin_nontemporal_store(v, dst);
            else
              *dst = v;
          }
        }
        continue;
      }
      // partial column range: per-element stores
      const int rl = r0 + l32;
      if (rl >= rows_valid) continue;
#pragma unroll
      for (int j = 0; j < CPR; ++j) {
        const int b = j / 4, g = j % 4;
        const int64_t c0 = c_base + j * 8 + half * 4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c0 + c >= nout) continue;
          if constexpr (GBWD) {
            float d1, d2;
            const float dac = to_f32(((const TO *)p.aux)[(m0 + rl) * p.ldaux + c0 + c]);
            glu_bwd_<EPI>(acc[a][0][4 * g + c], acc[a][1][4 * g + c], dac, p.beta1, p.beta2, d1, d2);
            C[(m0 + rl) * p.ldc + c0 + c] = from_f32<TO>(d1);
            C[(m0 + rl) * p.ldc + nout + c0 + c] = from_f32<TO>(d2);
          } else {
            const float v = GLU ? glu_<EPI>(acc[a][0][4 * g + c], acc[a][1][4 * g + c], p.beta1, p.beta2)
                                : acc[a][b][4 * g + c] * rs;
            C[(m0 + rl) * p.ldc + c0 + c] = from_f32<TO>(v);
          }
        }
      }
    }
    return;
  }
  const bool vec = (p.ldc % 4) == 0;
#pragma unroll
  for (int a = 0; a < TM; ++a) {
    const int rl = (a * WM + wm) * 32 + l32;
    if (rl >= rows_valid) continue;
    const int64_t grow = m0 + rl;
    const float rs = (EPI == EPI_ROWSCALE) ? p.row_scale[grow] : 1.0f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (is_glu_bwd<EPI>) {
        // gate backward: dx1 into columns [0, H), dx2 into [H, 2H) of the output
        const int64_t H = p.N / 2;
#pragma unroll
        for (int b = 0; b < TN; b += 2) {
          const int64_t h0 = (int64_t)nt * (BN / 2) + wn * (WTN / 2) + (b / 2) * 32 + g * 8 + half * 4;
          const TO *dap = (const TO *)p.aux + grow * p.ldaux + h0;
          TO *dst = C + grow * p.ldc + h0;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            if (h0 + c >= H) continue;
            float d1, d2;
            glu_bwd_<EPI>(acc[a][b][4 * g + c], acc[a][b + 1][4 * g + c], to_f32(dap[c]), p.beta1, p.beta2, d1, d2);
            dst[c] = from_f32<TO>(d1);
            dst[H + c] = from_f32<TO>(d2);
          }
        }
      } else if (is_glu<EPI>) {
#pragma unroll
        for (int b = 0; b < TN; b += 2) {
          const int64_t h0 = (int64_t)nt * (BN / 2) + wn * (WTN / 2) + (b / 2) * 32 + g * 8 + half * 4;
          float o[4];
#pragma unroll
          for (int c = 0; c < 4; ++c)
            o[c] = glu_<EPI>(acc[a][b][4 * g + c], acc[a][b + 1][4 * g + c], p.beta1, p.beta2);
          TO *dst = C + grow * p.ldc + h0;
          if (vec && h0 + 3 < p.N / 2) {
            store4(dst, o);
          } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
              if (h0 + c < p.N / 2) dst[c] = from_f32<TO>(o[c]);
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int64_t c0 = (int64_t)nt * BN + wn * WTN + b * 32 + g * 8 + half * 4;
          float o[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            float v = acc[a][b][4 * g + c];
            if (EPI == EPI_SIGMOID) {
              if (p.col_bias) v += p.col_bias[min(c0 + c, (int64_t)p.N - 1)];
              v = sigmoidf_(v);
            } else if (EPI == EPI_ROWSCALE) {
              v *= rs;
            }
            o[c] = v;
          }
          if (EPI == EPI_PARTIAL) {
            float *dst = (float *)p.C + ((int64_t)ks * p.M + grow) * p.ldc + c0;
            if (vec && c0 + 3 < p.N) {
              store4(dst, o);
            } else {
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (c0 + c < p.N) dst[c] = o[c];
            }
          } else {
            TO *dst = C + grow * p.ldc + c0;
            if (vec && c0 + 3 < p.N) {
              store4(dst, o);
            } else {
#pragma unroll
              for (int c = 0; c < 4; ++c)
                if (c0 + c < p.N) dst[c] = from_f32<TO>(o[c]);
            }
          }
        }
      }
    }
  }
}

// Tile configuration: BM x BN outputs per work-group of WM x WN waves; PF =
// how many K steps ahead the global loads run (PF register sets).  M subtiles of 32 rows are interleaved over the
// wave rows (wave wm owns subtiles wm, wm + WM, ...) so that a partially
// filled M tile still spreads its valid rows over the waves.
// Buffer resource over 4 GiB from base p (raw addressing: offsets below
// 2^32 - 1 are in range).  The address is made explicitly uniform, so the
// resource lives in scalar registers.
LMOE_DEV __amdgpu_buffer_rsrc_t uniform_rsrc(const void *p) {
  const uint64_t a = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc((void *)(((uint64_t)hi << 32) | lo), (short)0, -1, 0x00020000);
}
// s_waitcnt with lgkmcnt(0), expcnt untouched and vmcnt(N), N < 64
template <int N> LMOE_DEV void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (7 << 4) | (N & 15));
}
typedef __attribute__((address_space(3))) void lds_void_t;

// BDMA: both operands go straight from global memory into LDS (buffer loads
// with an LDS destination) instead of through registers: B through a ring of
// three stages, two steps ahead, A through two stages, one step ahead; a lane
// loads the 16-byte chunk of its row that the swizzle expects at its LDS slot.
// Buffer loads rather than the FLAT-encoded global-load-to-LDS: the compiler
// counts those as possible LDS accesses that complete out of order and turns
// every later LDS wait into a full lgkmcnt(0).  With no LDS stores left in the
// K loop, each step waits only for the loads of the next one (an LDS store
// after such loads would make the compiler wait for all of them).
template <typename T, typename TO, int BM, int BN, int WM, int WN, int PF, int EPI, bool GATHER, bool GROUPED,
          bool BDMA = false, bool BKN = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs p) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTN = BN / WN;
  constexpr int TM = BM / WM / 32, TN = WTN / 32;
  constexpr int BKE = 128 / (int)sizeof(T);
  constexpr int CPL = Mma<T>::CPL;
  constexpr int NG = BKE / 16;
  constexpr int RPP = NT / 8;  // rows covered per load pass (8 threads x 16 B per row)
  constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
  constexpr int EPT = 16 / (int)sizeof(T);  // elements per 16-B chunk
  constexpr int NSET = PF;  // B register sets: B(j) lives in set j % PF
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of the load pass");
  static_assert(BM % (32 * WM) == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(!is_glu<EPI> || TN % 2 == 0, "GLU needs W1/W2 subtile pairs");
  static_assert(PF >= 1 && PF <= 4, "prefetch distance");
  static_assert(NG == 2 || NG == 4, "16-K groups per 128-byte K step");
  static_assert(!BDMA || (PF == 2 && RPP == 64 && EPI != EPI_PARTIAL), "load to LDS: two-step pipeline, 8 waves");
  // BKN: B stored [K, N]; each thread loads KR = B_LD rows of one 16-byte column
  // chunk and writes them transposed (through registers, so not with BDMA)
  static_assert(!BKN || (!BDMA && !is_glu<EPI> && EPI != EPI_PARTIAL && (NT == 256 || NT == 512) && BN == 256),
                "B stored [K, N]: register-staged, plain epilogues, 256-column tiles");
  static_assert(!BKN || B_LD * (NT / 64) * 64 * EPT == BKE * BN, "B stored [K, N]: one column chunk per thread");
  constexpr int NSB = BDMA ? 3 : 2;  // LDS stages of B
  constexpr bool STAGED = StagedStore<TO, EPI, WTN, TN>::value;
  static_assert(!BDMA || !STAGED || (NT / 64) * STAGE_BYTES_PER_WAVE <= BN * 128, "staging fits one B stage");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char *const sA0 = smem;
  unsigned char *const sB0 = smem + 2 * BM * 128;
  // wave-private epilogue staging area (only for the staged-store epilogue); with
  // BDMA it lives in the B stage the tile's last step has just consumed
  unsigned char *sE = smem + 2 * (BM + BN) * 128 + (threadIdx.x >> 6) * STAGE_BYTES_PER_WAVE;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform by construction; readfirstlane lets the compiler keep it (and
  // everything derived from it) in scalar registers, so per-subtile tests branch
  // on SCC instead of masking lanes
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // Lane-derived indices are re-derived from an opaque copy of the thread id
  // at the start of every tile, so the compiler cannot hoist the many LDS and
  // store addresses built from them out of the tile loop (they would then stay
  // live through the epilogue and spill).
  int half = lane >> 5, l32 = lane & 31;
  int lrow = tid >> 3, lchunk = tid & 7;
  // BDMA: the chunk this lane loads so that its LDS slot (lane & 7 of row lrow)
  // holds what swz() expects: slot ^ (row & 7) ^ ((row >> 3) & 1)
  int lbc = (tid & 7) ^ ((tid >> 3) & 7) ^ ((tid >> 6) & 1);
  // BKN: this thread's column chunk (kn_nb: EPT columns) and K group (kn_kg: B_LD
  // rows), chosen so that the loads of a wave cover whole 512-byte row segments
  // and the transposed LDS writes are free of bank conflicts under swz_kn:
  //   bf16, 8 waves: 8 chunks x 2 K groups per 16 lanes; bf16, 4 waves: 8 chunks
  //   per 8 lanes; fp32: lane = chunk, wave = K group
  int kn_nb = 0, kn_kg = 0;
  if constexpr (BKN) {
    if constexpr (sizeof(T) == 2 && NT == 512) {
      kn_nb = (lane & 7) + 8 * (lane >> 4);
      kn_kg = 2 * wave + ((lane >> 3) & 1);
    } else if constexpr (sizeof(T) == 2) {
      kn_nb = (lane & 7) + 8 * ((lane >> 3) & 3);
      kn_kg = 2 * wave + (lane >> 5);
    } else {
      kn_nb = lane;
      kn_kg = wave;
    }
  }

  // ---- persistent walk over the logical tiles.  Each XCD (work-groups are
  // dispatched round-robin over the 8 XCDs) takes one contiguous range of
  // logical tiles, so the tiles that share A rows (one expert's N tiles, or a
  // group of dense M tiles) meet in that XCD's L2.  The first `per` tiles of a
  // range go one to each of the XCD's work-groups.  Dense GEMMs then walk their
  // range with a stride; grouped GEMMs (tiles of uneven cost) take the rest in
  // order from a per-XCD counter, so an expert's N tiles start close together
  // (its gathered rows are fetched into L2 once) and a work-group that finishes
  // early takes more; once its own range is used up it takes from the other
  // XCDs' ranges.  Thread 0 takes the tile after next at the start of a tile
  // and publishes it through LDS after the first K step, so the next tile is
  // always known when its loads are issued.
  const int nvalid = GROUPED ? min(*p.ntiles, p.tiles_m) * p.tiles_n : p.n_logical;
  const int nx = (gridDim.x % 8 == 0) ? 8 : 1;
  const int per = gridDim.x / nx;
  const int chunk = (nvalid + nx - 1) / nx;
  const int xcd = blockIdx.x % nx;
  const int lt_end = min(nvalid, (xcd + 1) * chunk);
  int lt = xcd * chunk + blockIdx.x / nx;
  if (lt >= lt_end) return;
  const bool dyn = GROUPED && p.sched != nullptr;
  int *const qslot = (int *)(smem + (BDMA ? 2 * BM * 128 + NSB * BN * 128
                                          : 2 * (BM + BN) * 128 + (STAGED ? (NT / 64) * STAGE_BYTES_PER_WAVE : 0)));
  int steal = 0;  // thread 0: ranges (own XCD's first) found used up
  auto grab = [&]() -> int {
    while (steal < nx) {
      const int xi = (xcd + steal) % nx;
      const int j = xi * chunk + per + atomicAdd(&p.sched[xi], 1);
      if (j < min(nvalid, (xi + 1) * chunk)) return j;
      ++steal;
    }
    return -1;
  };
  int q_next = -1;  // dyn: the tile after the current one (-1: none)
  if (GROUPED && dyn) {
    if (tid == 0) {
      qslot[0] = grab();
      qslot[1] = -1;
    }
    __syncthreads();
    q_next = qslot[0];
    __syncthreads();
  }
  int tile_par = 0;  // dyn: parity of the tile count, selects the LDS slot

  const int nk_all = p.K / BKE;
  auto decode = [&](int l) { return decode_tile<T, TO, BM, GROUPED>(p, l, nk_all); };

  // ---- per-thread source rows of the tile being loaded (32-bit row indices;
  // addresses are formed per K step).  Rows past the valid range are clamped
  // onto a valid row: they only feed output rows / columns that are never
  // stored, and unconditional loads keep the K loop free of branches (whose
  // joins force full vmcnt waits).
  int a_row[A_LD];
  int b_row[B_LD];  // row of B (GLU: hidden unit)
  bool b_w2[B_LD];  // GLU / split-K: row comes from B2
  const T *lb1, *lb2;  // B (and B2) of the tile being loaded, at this thread's 16-B chunk
  int lkbeg;        // first K step
  // BDMA: buffer resources of A and of the tile's B (or B2) matrix this wave
  // loads from, and the byte offset of this lane's chunk of each B row it loads
  // (the K offset goes in soffset)
  const __amdgpu_buffer_rsrc_t rsA = uniform_rsrc(p.A);
  __amdgpu_buffer_rsrc_t rsB = rsA;
  int b_vo[B_LD];  // (int: with an unsigned array here the host pass silently drops the kernel)
  // (BDMA: out[i] is the byte offset of the lane's chunk of row i from A,
  // which the host keeps below 4 GiB)
  auto rows_of = [&](const TileI &t, int (&out)[A_LD]) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int r = min(lrow + i * RPP, t.rows - 1);
      const int row = GATHER ? p.a_rows[t.m0 + r] : (int)(t.m0 + r);
      out[i] = BDMA ? (int)((uint32_t)row * (uint32_t)(p.lda * sizeof(T)) + (uint32_t)lbc * 16u) : row;
    }
  };
  auto set_b = [&](const TileI &t) {
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int br = lrow + i * RPP;
      if (is_glu<EPI>) {
        const int wcol = br / WTN, within = br % WTN, j = within / 32;
        const int row = t.nt * (BN / 2) + wcol * (WTN / 2) + (j / 2) * 32 + (br & 31);
        b_row[i] = min(row, p.N / 2 - 1);
        b_w2[i] = (j & 1) != 0;
      } else if (EPI == EPI_PARTIAL) {
        const int row = min(t.nt * BN + br, p.N - 1);
        b_w2[i] = row >= p.b_split_row;
        b_row[i] = b_w2[i] ? row - p.b_split_row : row;
      } else {
        b_row[i] = min(t.nt * BN + br, p.N - 1);
        b_w2[i] = false;
      }
    }
    const int bc = BDMA ? lbc : lchunk;
    lb1 = (const T *)t.B + bc * EPT;
    lb2 = ((is_glu<EPI> || EPI == EPI_PARTIAL) && t.B2) ? (const T *)t.B2 + bc * EPT : lb1;
    if constexpr (BKN) {  // the thread's column chunk (clamped onto the last one: never stored)
      const int col = min(t.nt * BN + kn_nb * EPT, p.N - EPT);
      lb1 = (const T *)t.B + col;
      lb2 = t.B2 ? (const T *)t.B2 + col : lb1;
    }
    if constexpr (BDMA) {
#pragma unroll
      for (int i = 0; i < B_LD; ++i) b_vo[i] = (int)((uint32_t)b_row[i] * (uint32_t)(p.ldb * sizeof(T)) + (uint32_t)lbc * 16u);
      // GLU: the 8 rows of each of the wave's loads lie in one 32-row block, of W1
      // or W2, and adding 64 rows (a load pass) keeps the block's parity, so the
      // wave reads one matrix throughout
      const bool w2 = is_glu<EPI> && ((((8 * wave) % WTN) / 32) & 1) != 0;
      rsB = uniform_rsrc((w2 && t.B2) ? t.B2 : t.B);
    }
    lkbeg = __builtin_amdgcn_readfirstlane(t.kbeg);  // uniform (a buffer offset operand)
  };
  const T *const Abase = (const T *)p.A + lchunk * EPT;

  // register sets of staged global loads (see the pipeline below)
  u32x4 ra[NSET][A_LD], rb[NSET][B_LD];
  const bool kbatch = p.kb_len != p.K;

  auto gloadB = [&](auto SETC, int kt) {
    constexpr int S = decltype(SETC)::value;
    const int k0 = (lkbeg + kt) * BKE;
    if constexpr (BKN) {  // rows k0 + kg * B_LD + i of B (K rows past kb_len: of B2)
#pragma unroll
      for (int i = 0; i < B_LD; ++i) {
        const int k = k0 + kn_kg * B_LD + i;
        const bool second = kbatch && k >= (int)p.kb_len;
        const u32x4 *bp = (const u32x4 *)((second ? lb2 : lb1) + (int64_t)(second ? k - (int)p.kb_len : k) * p.ldb);
        rb[S][i] = GROUPED ? __builtin_nontemporal_load(bp) : *bp;
      }
      return;
    }
    int64_t boff = k0;
    if (kbatch) {  // uniform; only a K-batched B (several matrices side by side along K)
      const int s = k0 / (int)p.kb_len;
      boff = (int64_t)s * p.kb_stride + (k0 - s * (int)p.kb_len);
    }
    // Expert weights (grouped) are streamed once per forward: non-temporal
    // loads keep them from displacing the gathered rows and other reused data
    // in the caches.  Dense B is re-read by every M tile and stays cached.
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const u32x4 *bp = (const u32x4 *)((b_w2[i] ? lb2 : lb1) + (int64_t)b_row[i] * p.ldb + boff);
      rb[S][i] = GROUPED ? __builtin_nontemporal_load(bp) : *bp;
    }
  };
  // BDMA: B of tile step kt into the LDS stage of global step g; instruction i of
  // wave w writes tile rows 8w + 64i .. +7 (1 KB), one row chunk per lane
  // (B is one matrix along K here: no K batches, checked at launch)
  auto dmaBr = [&](auto I0, auto I1, int kt, int g) {
    const uint32_t so = (uint32_t)((lkbeg + kt) * BKE * (int)sizeof(T));
    unsigned char *dst = sB0 + (g % NSB) * BN * 128 + wave * 8 * 128;
#pragma unroll
    for (int i = decltype(I0)::value; i < decltype(I1)::value; ++i) {
      // expert weights are streamed once (non-temporal); dense B is re-read by other M tiles
      if constexpr (GROUPED)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void_t *)(dst + i * RPP * 128), 16, (uint32_t)b_vo[i], so, 0, 2);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void_t *)(dst + i * RPP * 128), 16, (uint32_t)b_vo[i], so, 0, 0);
    }
  };
  auto dmaB = [&](int kt, int g) { dmaBr(IC<0>{}, IC<B_LD>{}, kt, g); };
  // BDMA: A of tile step kt into the LDS stage of global step g (rows as for B)
  auto dmaA = [&](int kt, int g) {
    const uint32_t so = (uint32_t)((lkbeg + kt) * BKE * (int)sizeof(T));
    unsigned char *dst = sA0 + (g & 1) * BM * 128 + wave * 8 * 128;
#pragma unroll
    for (int i = 0; i < A_LD; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void_t *)(dst + i * RPP * 128), 16, (uint32_t)a_row[i], so, 0, 0);
  };
  auto gloadA = [&](auto SETC, int kt) {
    constexpr int S = decltype(SETC)::value;
    const int64_t k0 = (int64_t)(lkbeg + kt) * BKE;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[S][i] = *(const u32x4 *)(Abase + (int64_t)a_row[i] * p.lda + k0);
  };
  auto lstore = [&](auto SETC, int buf) {
    constexpr int S = decltype(SETC)::value;
    unsigned char *sA = sA0 + buf * BM * 128;
    unsigned char *sB = sB0 + buf * BN * 128;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(u32x4 *)(sA + swz(lrow + i * RPP, lchunk)) = ra[S][i];
    if constexpr (BKN) {
      // column j of the chunk is tile row kn_nb * EPT + j; its B_LD K values
      // (rows kn_kg * B_LD .. of the step) are element j of each loaded chunk
#pragma unroll
      for (int j = 0; j < EPT; ++j) {
        const int r = kn_nb * EPT + j;
        if constexpr (sizeof(T) == 2) {
          // bf16 pairs (k, k + 1) of column j: halves j & 1 of word j >> 1
          const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
          uint32_t w[B_LD / 2];
#pragma unroll
          for (int q = 0; q < B_LD / 2; ++q)
            w[q] = __builtin_amdgcn_perm(rb[S][2 * q + 1][j >> 1], rb[S][2 * q][j >> 1], sel);
          if constexpr (B_LD == 4) {  // 8 bytes: half kn_kg & 1 of chunk kn_kg >> 1
            u32x2 v2 = {w[0], w[1]};
            *(u32x2 *)(sB + swz_kn(r, kn_kg >> 1) + (kn_kg & 1) * 8) = v2;
          } else {
            u32x4 v4 = {w[0], w[1], w[2], w[3]};
            *(u32x4 *)(sB + swz_kn(r, kn_kg)) = v4;
          }
        } else {
#pragma unroll
          for (int h = 0; h < B_LD / 4; ++h) {
            u32x4 v4 = {rb[S][4 * h][j], rb[S][4 * h + 1][j], rb[S][4 * h + 2][j], rb[S][4 * h + 3][j]};
            *(u32x4 *)(sB + swz_kn(r, kn_kg * (B_LD / 4) + h)) = v4;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < B_LD; ++i) *(u32x4 *)(sB + swz(lrow + i * RPP, lchunk)) = rb[S][i];
    }
  };

  f32x16 acc[TM][TN];
  bool skip_last = false;  // grouped: this wave's last M subtile is all padding in the current tile

  // One K step from LDS buffer `buf`: the fragments of 16-K group g+1 are read
  // while the MFMAs of group g run (two fragment register sets).
  auto compute = [&](int buf, const unsigned char *sB, auto &&mid) {
    const unsigned char *sA = sA0 + buf * BM * 128;
    u32x4 af[2][TM][CPL], bfg[2][TN][CPL];
    auto frags = [&](auto GC, auto SC) {
      constexpr int g = decltype(GC)::value, f = decltype(SC)::value;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int r = wn * WTN + b * 32 + l32;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int ch = g * 2 * CPL + half * CPL + c;
          bfg[f][b][c] = *(const u32x4 *)(sB + (BKN ? swz_kn(r, ch) : swz(r, ch)));
        }
      }
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        if (a == TM - 1 && skip_last) continue;
        const int r = (a * WM + wm) * 32 + l32;
#pragma unroll
        for (int c = 0; c < CPL; ++c) af[f][a][c] = *(const u32x4 *)(sA + swz(r, g * 2 * CPL + half * CPL + c));
      }
    };
    auto mma = [&](auto SC) {
      constexpr int f = decltype(SC)::value;
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        if (a == TM - 1 && skip_last) continue;
#pragma unroll
        for (int b = 0; b < TN; ++b) Mma<T>::run(bfg[f][b], af[f][a], acc[a][b]);
      }
    };
    // interleave: one MFMA, then one LDS read of the next group's fragments
    auto interleave = [&]() {
      constexpr int NR = (TN + TM) * CPL, NM = TM * TN * (CPL == 1 ? 1 : 8);
#pragma unroll
      for (int i = 0; i < (NR < NM ? NR : NM); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
      }
    };
    frags(IC<0>{}, IC<0>{});
    if (NG > 1) frags(IC<1 % NG>{}, IC<1>{});
    mma(IC<0>{});
    mid();  // e.g. the LDS store of the next step, overlapped with these MFMAs
    if (NG > 2) {
      frags(IC<2 % NG>{}, IC<0>{});
      interleave();
    }
    if (NG > 1) mma(IC<1>{});
    if (NG > 3) {
      frags(IC<3 % NG>{}, IC<1>{});
      interleave();
    }
    if (NG > 2) mma(IC<0>{});
    if (NG > 3) mma(IC<1>{});
  };

  // BDMA K steps run as fenced phases over two fragment register sets: phase i
  // issues the LDS reads of 16-K group i + 1 and then the MFMAs of group i (whose
  // reads the previous phase issued), and the group-0 reads of the next step are
  // issued right after the barrier that makes its operands visible, ahead of the
  // MFMAs of the step's last group.  The fences keep the compiler from pulling
  // reads next to the MFMAs that consume them, so each wait covers only reads
  // issued a full phase earlier.  SK (a compile-time flag, chosen once per tile)
  // drops the wave's last M subtile when it holds only padding rows.
  u32x4 fa[2][TM][CPL], fb[2][TN][CPL];
  auto rd = [&](auto SKC, auto GC, auto SC, int oa, int ob) {
    constexpr bool SK = decltype(SKC)::value != 0;
    constexpr int g = decltype(GC)::value, f = decltype(SC)::value;
    const unsigned char *sA = sA0 + oa, *sB = sB0 + ob;
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int r = wn * WTN + b * 32 + l32;
#pragma unroll
      for (int c = 0; c < CPL; ++c) fb[f][b][c] = *(const u32x4 *)(sB + swz(r, g * 2 * CPL + half * CPL + c));
    }
#pragma unroll
    for (int a = 0; a < TM - (SK ? 1 : 0); ++a) {
      const int r = (a * WM + wm) * 32 + l32;
#pragma unroll
      for (int c = 0; c < CPL; ++c) fa[f][a][c] = *(const u32x4 *)(sA + swz(r, g * 2 * CPL + half * CPL + c));
    }
  };
  auto mm = [&](auto SKC, auto SC) {
    constexpr bool SK = decltype(SKC)::value != 0;
    constexpr int f = decltype(SC)::value;
#pragma unroll
    for (int a = 0; a < TM - (SK ? 1 : 0); ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) Mma<T>::run(fb[f][b], fa[f][a], acc[a][b]);
  };
  // (dma issues ND global-to-LDS loads of later steps, one after each of the
  // phase's first MFMAs, so no wave stalls on a burst of them while its MFMAs
  // could run)
  auto phase = [&](auto SKC, auto GC, auto SN, auto SM, int oa, int ob, auto &&dma, auto NDC) {
    constexpr bool SK = decltype(SKC)::value != 0;
    constexpr int NR = (TN + TM - (SK ? 1 : 0)) * CPL;
    constexpr int NM = TN * (TM - (SK ? 1 : 0)) * (sizeof(T) == 4 ? 8 : 1);
    constexpr int ND = decltype(NDC)::value;
    static_assert(ND <= NM, "one load per MFMA at most");
    rd(SKC, GC, SN, oa, ob);
    mm(SKC, SM);
    dma();
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // the reads first
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // a load
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - ND, 0);  // the other MFMAs
    __builtin_amdgcn_sched_barrier(0);
  };

  // Pipeline (one barrier per K step).
  //  PF == 1: A(kt+1), B(kt+1) are loaded at the start of step kt and stored to
  //           the other LDS buffer after the step's MFMAs.
  //  PF >= 2: A(j), B(j) live in register set j % PF and are loaded PF steps
  //           ahead; during step kt the loads of step kt+PF are issued first,
  //           then the LDS store of step kt+1 (whose loads were issued PF-1
  //           steps earlier, so vmcnt only waits for them) runs in the middle
  //           of the step's MFMAs instead of after them.
  // Across tiles: when every tile's number of K steps is a multiple of 2 and
  // of PF (p.xpf), the last steps of a tile already load the first steps of
  // the work-group's next tile, so those loads are in flight while the tile's
  // epilogue stores run; otherwise each tile starts with its own prologue.
  int gbase = 0;  // BDMA: global step index of the current tile's step 0
  auto prologue = [&](int nk) {
    if constexpr (BDMA) {
      dmaA(0, gbase);
      dmaB(0, gbase);
      if (1 < nk) dmaB(1, gbase + 1);
      wait_vm_lgkm0<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      return;
    }
    gloadA(IC<0>{}, 0);
    gloadB(IC<0>{}, 0);
    if (PF > 1 && 1 < nk) {
      gloadA(IC<1 % NSET>{}, 1);
      gloadB(IC<1 % NSET>{}, 1);
    }
    if (PF > 2 && 2 < nk) {
      gloadA(IC<2 % NSET>{}, 2);
      gloadB(IC<2 % NSET>{}, 2);
    }
    if (PF > 3 && 3 < nk) {
      gloadA(IC<3 % NSET>{}, 3);
      gloadB(IC<3 % NSET>{}, 3);
    }
    lstore(IC<0>{}, 0);
    __syncthreads();
  };

  TileI cur = decode(lt);
  rows_of(cur, a_row);
  set_b(cur);
  prologue(cur.nk);
  const bool xpf = p.xpf != 0;

  while (true) {
    {
      int t_o = threadIdx.x;
      asm volatile("" : "+v"(t_o));
      half = (t_o >> 5) & 1;
      l32 = t_o & 31;
      lrow = t_o >> 3;
      lchunk = t_o & 7;
      lbc = (t_o & 7) ^ ((t_o >> 3) & 7) ^ ((t_o >> 6) & 1);
    }
    const int lt_next = dyn ? q_next : lt + per;
    const bool has_next = dyn ? lt_next >= 0 : lt_next < lt_end;
    int grabbed = -1;  // thread 0: the tile after lt_next
    if (GROUPED && dyn && tid == 0) grabbed = has_next ? grab() : -1;
    const bool xnext = xpf && has_next;
    TileI nxt = cur;
    int n_row[A_LD];
    if (has_next) nxt = decode(lt_next);
    if (xnext) rows_of(nxt, n_row);
    const int nk = cur.nk;
    // Grouped tiles are cut to their expert's rows, so the last M tile of an
    // expert is often short: when this wave's last 32-row subtile holds only
    // padding rows (never stored), its fragment reads and MFMAs are skipped
    // (a wave-uniform branch; with ~146 rows per 192-row tile this removes a
    // sixth of the routed MFMAs)
    skip_last = GROUPED && TM > 1 && __builtin_amdgcn_readfirstlane(((TM - 1) * WM + wm) * 32 >= cur.rows ? 1 : 0) != 0;

#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

    // loads for step j of this tile, or (j >= nk) step j - nk of the next one
    auto loads = [&](auto SETC, auto CHECKC, int j) {
      constexpr bool CHECK = decltype(CHECKC)::value != 0;
      if (!CHECK || j < nk) {
        gloadA(SETC, j);
        gloadB(SETC, j);
      } else if (xnext) {
        if (j == nk) {  // first load of the next tile: switch the source rows
#pragma unroll
          for (int i = 0; i < A_LD; ++i) a_row[i] = n_row[i];
          set_b(nxt);
        }
        gloadA(SETC, j - nk);
        gloadB(SETC, j - nk);
      }
    };
    auto step = [&](auto SETC, auto CHECKC, int kt) {
      constexpr int S = decltype(SETC)::value;  // == kt % NSET
      constexpr bool CHECK = decltype(CHECKC)::value != 0;
      const bool st_next = !CHECK || kt + 1 < nk || xnext;
      const unsigned char *sBk = sB0 + (kt & 1) * BN * 128;
      if (PF == 1) {
        loads(IC<0>{}, CHECKC, kt + 1);
        compute(kt & 1, sBk, [] {});
        if (st_next) lstore(IC<0>{}, (kt + 1) & 1);
      } else {
        loads(IC<S>{}, CHECKC, kt + PF);
        compute(kt & 1, sBk, [&] {
          if (st_next) lstore(IC<(S + 1) % NSET>{}, (kt + 1) & 1);
        });
      }
      if (GROUPED && dyn && kt == 0 && tid == 0) qslot[tile_par] = grabbed;
      __syncthreads();
    };
    // BDMA: one K step (see the phase comment above)
    auto pstep = [&](auto SKC, auto CHECKC, int kt) {
      constexpr bool CHECK = decltype(CHECKC)::value != 0;
      const int g = gbase + kt;
      // A of step kt + 1 and B of step kt + 2 (past the tile's end: the next
      // tile's first steps, whose source rows are switched in just before)
      const int ja = kt + 1, jb = kt + 2;
      const bool a_iss = !CHECK || ja < nk || xnext;
      const bool b_iss = !CHECK || jb < nk || xnext;
      if (CHECK && ja == nk && xnext) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) a_row[i] = n_row[i];
      }
      const int ka = (!CHECK || ja < nk) ? ja : ja - nk;
      const int kb = (!CHECK || jb < nk) ? jb : jb - nk;
      auto dA = [&] {
        if (a_iss) dmaA(ka, g + 1);
      };
      // (the B rows switch after the A loads, which still use this tile's K start)
      auto dB0 = [&] {
        if (CHECK && jb == nk && xnext) set_b(nxt);
        if (b_iss) dmaBr(IC<0>{}, IC<B_LD / 2>{}, kb, g + 2);
      };
      auto dB1 = [&] {
        if (b_iss) dmaBr(IC<B_LD / 2>{}, IC<B_LD>{}, kb, g + 2);
      };
      const int oa = (g & 1) * BM * 128, ob = (g % NSB) * BN * 128;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NG == 4) {
        phase(SKC, IC<1>{}, IC<1>{}, IC<0>{}, oa, ob, dA, IC<A_LD>{});
        phase(SKC, IC<2>{}, IC<0>{}, IC<1>{}, oa, ob, dB0, IC<B_LD / 2>{});
        phase(SKC, IC<3>{}, IC<1>{}, IC<0>{}, oa, ob, dB1, IC<B_LD - B_LD / 2>{});
      } else {
        phase(SKC, IC<1>{}, IC<1>{}, IC<0>{}, oa, ob, [&] { dA(); dB0(); dB1(); }, IC<A_LD + B_LD>{});
      }
      if (GROUPED && dyn && kt == 0 && tid == 0) qslot[tile_par] = grabbed;
      // A and B of step kt + 1 must be in LDS (only this step's B loads, if
      // any, were issued after them) and this step's reads done
      if (b_iss) wait_vm_lgkm0<B_LD>();
      else wait_vm_lgkm0<0>();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (!CHECK || kt + 1 < nk) rd(SKC, IC<0>{}, IC<0>{}, ((g + 1) & 1) * BM * 128, ((g + 1) % NSB) * BN * 128);
      mm(SKC, IC<1>{});
      __builtin_amdgcn_sched_barrier(0);
    };
    // NSET consecutive steps (register set indices known at compile time)
    auto steps = [&](auto CHECKC, int kt) {
      constexpr bool CHECK = decltype(CHECKC)::value != 0;
      step(IC<0>{}, CHECKC, kt);
      if (NSET > 1 && (!CHECK || kt + 1 < nk)) step(IC<1 % NSET>{}, CHECKC, kt + 1);
      if (NSET > 2 && (!CHECK || kt + 2 < nk)) step(IC<2 % NSET>{}, CHECKC, kt + 2);
      if (NSET > 3 && (!CHECK || kt + 3 < nk)) step(IC<3 % NSET>{}, CHECKC, kt + 3);
    };
    // Every subtile is computed, valid rows or not (rows past the valid range
    // hold copies of a valid row and are never stored): the K loop stays free
    // of branches, and the MFMA time of a full tile is still below the time to
    // stream its weights.
    if constexpr (BDMA) {
      auto kloop = [&](auto SKC) {
        if (nk > 0) rd(SKC, IC<0>{}, IC<0>{}, (gbase & 1) * BM * 128, (gbase % NSB) * BN * 128);
        int kt = 0;
        for (; kt + 2 < nk; ++kt) pstep(SKC, IC<0>{}, kt);
        for (; kt < nk; ++kt) pstep(SKC, IC<1>{}, kt);
      };
      if (skip_last) kloop(IC<1>{});
      else kloop(IC<0>{});
    } else {
      int kt = 0;
      for (; kt + NSET + PF <= nk; kt += NSET) steps(IC<0>{}, kt);
      for (; kt < nk; kt += NSET) steps(IC<1>{}, kt);
    }

    // published after step 0 of this tile; the slot is rewritten two tiles later,
    // past a barrier every thread reaches only after this read.  A K-range tile
    // without K steps (an expert with no rows) has no step 0: it publishes here
    // (nk is uniform over the work-group, so the barrier is too).
    if (GROUPED && dyn) {
      if (nk == 0) {
        if (tid == 0) qslot[tile_par] = grabbed;
        __syncthreads();
      }
      q_next = qslot[tile_par];
      tile_par ^= 1;
    }

    // ---- epilogue
    // (a K-range tile may have no K step at all: its zero tile is still stored)
    if constexpr (BDMA) sE = sB0 + ((gbase + nk + NSB - 1) % NSB) * BN * 128 + (threadIdx.x >> 6) * STAGE_BYTES_PER_WAVE;
    store_tile<TO, EPI, BN, WTN, WM, TM, TN>(p, cur.C, acc, cur.m0, cur.rows, cur.nt, cur.ks, wm, wn, half, l32, sE);
    if constexpr (BDMA && STAGED) {
      // the next tile's first step loads B into the stage used for staging
      __builtin_amdgcn_s_waitcnt((7 << 4) | 0xF | (3 << 14));  // lgkmcnt(0) only
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    gbase += nk;

    if (!has_next) break;
    lt = lt_next;
    cur = nxt;
    if (!xpf) {
      rows_of(cur, a_row);
      set_b(cur);
      prologue(cur.nk);
    }
  }
}

// Split-K finalize: out = epilogue(sum over splits of the fp32 partials).
// The gated epilogues read the stacked layout: W1 products in columns [0, H), W2 in [H, 2H).
template <typename TO, int EPI>
__global__ __launch_bounds__(256) void splitk_finalize_kernel(const float *__restrict__ part, int splits, int M,
                                                              int Np, TO *__restrict__ out, int64_t ldo,
                                                              const float *__restrict__ col_bias, float beta1,
                                                              float beta2) {
  const int Nout = (is_glu<EPI>) ? Np / 2 : Np;
  const int64_t total = (int64_t)M * Nout;
  const int64_t plane = (int64_t)M * Np;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int m = (int)(i / Nout), c = (int)(i % Nout);
    const float *pp = part + (int64_t)m * Np + c;
    float v = 0.0f;
    for (int sp = 0; sp < splits; ++sp) v += pp[sp * plane];
    if (is_glu<EPI>) {
      float v2 = 0.0f;
      for (int sp = 0; sp < splits; ++sp) v2 += pp[sp * plane + Nout];
      v = glu_<EPI>(v, v2, beta1, beta2);
    } else if (EPI == EPI_SIGMOID) {
      if (col_bias) v += col_bias[c];
      v = sigmoidf_(v);
    }
    out[(int64_t)m * ldo + c] = from_f32<TO>(v);
  }
}

}  // namespace lmoe
