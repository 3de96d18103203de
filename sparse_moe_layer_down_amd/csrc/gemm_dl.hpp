// Dense bf16 GEMM with both operands loaded straight into LDS (the gfx950
// global-load-to-LDS path): C[M, N] = A[M, K] . B[N, K]^T, fp32 accumulation.
//
// 256 x 256 output tile on four waves (2 x 2), one wave per SIMD, each wave
// owning 128 x 128 outputs (4 x 4 blocks of 32 x 32), so every 16-byte
// fragment read from LDS feeds two MFMAs (an 8-wave 256 x 256 tile reads 0.75
// fragments per MFMA).  No register staging: a K step (32 elements, 64 bytes
// of each of the tile's 512 rows) is written into LDS by 8 load instructions
// per wave, each covering 16 rows; a lane fetches the 16-byte chunk of its row
// that the swizzle of the fragment reads expects at its LDS slot.  NS LDS
// stages: the loads run NS - 1 steps ahead, and the barrier closing a step
// waits only for the loads of the step after it.
#pragma once
#include "gemm.hpp"

namespace lmoe {

typedef __attribute__((address_space(3))) void lds_void_t;

// LDS address of 16-byte chunk c (0..3) of row r in a stage of 64-byte rows:
// the chunk is XOR-swizzled by (r >> 1) & 3 so that a fragment read (one chunk
// column, 8 consecutive rows per LDS pass) covers all 32 banks.
LMOE_DEV int swz64(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 3)) << 4); }

// s_waitcnt with lgkmcnt(0), expcnt untouched and vmcnt(N), N < 64
template <int N> LMOE_DEV void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (7 << 4) | (N & 15));
}

template <typename TO, int EPI>
__global__ __launch_bounds__(256) void gemm_dl_kernel(GemmArgs p) {
  constexpr int BM = 256, BN = 256, WM = 2, WN = 2;
  constexpr int WTN = BN / WN, TM = BM / WM / 32, TN = WTN / 32;
  constexpr int BKE = 32;                       // bf16 elements per K step (64 bytes of a row)
  constexpr int NS = 4;                         // LDS stages
  constexpr int STAGE = (BM + BN) * 64;         // bytes of one stage
  constexpr int NLD = (BM + BN) / 16 / 4;       // 16-row load instructions per wave per step
  constexpr int NLA = BM / 16 / 4;              // of which rows of A
  static_assert(TM == 4 && TN == 4 && NLD == 8, "four 128 x 128 wave tiles");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;

  // persistent walk: each XCD takes one contiguous range of the logical tiles
  // (groups of 8 M tiles walked down before across share their B rows in L2)
  const int nvalid = p.n_logical;
  const int nx = (gridDim.x % 8 == 0) ? 8 : 1;
  const int per = gridDim.x / nx;
  const int chunk = (nvalid + nx - 1) / nx;
  const int xcd = blockIdx.x % nx;
  const int lt_end = min(nvalid, (xcd + 1) * chunk);
  int lt = xcd * chunk + blockIdx.x / nx;
  if (lt >= lt_end) return;
  const int nk = p.K / BKE;

  // Load instruction i of this wave covers tile rows 16j .. 16j + 15, j = wave + 4i
  // (j < BM / 16: rows of A, else rows of B).  Lane -> row 16j + (lane >> 2) and
  // LDS slot lane & 3, which holds chunk slot ^ ((row >> 1) & 3) of the row;
  // (row >> 1) & 3 = (lane >> 3) & 3.
  const int lr = lane >> 2;
  const int lc = (lane & 3) ^ ((lane >> 3) & 3);
  // per tile: base pointers of its A and B rows, and per instruction the 32-bit
  // element offset of this lane's source chunk from them
  const bf16 *abase, *bbase;
  int src[NLD];
  auto set_src = [&](const TileI &t) {
    abase = (const bf16 *)p.A + t.m0 * p.lda;
    bbase = (const bf16 *)p.B + (int64_t)t.nt * BN * p.ldb;
    const int rows_a = (int)min((int64_t)BM, (int64_t)p.M - t.m0);
    const int rows_b = min(BN, p.N - t.nt * BN);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int j = wave + 4 * i;
      if (i < NLA)
        src[i] = min(16 * j + lr, rows_a - 1) * (int)p.lda + lc * 8;  // rows past M feed outputs never stored
      else
        src[i] = min(16 * (j - BM / 16) + lr, rows_b - 1) * (int)p.ldb + lc * 8;
    }
  };
  auto issue = [&](int kstep) {
    const int k0 = kstep * BKE;
    unsigned char *const base = smem + (kstep % NS) * STAGE;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int j = wave + 4 * i;
      const bf16 *g = (i < NLA ? abase : bbase) + (src[i] + k0);
      __builtin_amdgcn_global_load_lds((const void *)g, (lds_void_t *)(base + j * 1024), 16, 0, 0);
    }
  };
  // The barrier closing a step: this wave's loads of the next step are in LDS
  // (the N load instructions issued after them may still be in flight) and its
  // fragment reads are done; the memory clobbers keep the compiler from moving
  // LDS accesses across it.
  auto close_step = [&](auto NC) {
    wait_vm_lgkm0<decltype(NC)::value>();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x16 acc[TM][TN];
  // one K step: 2 groups of 16 K; the fragments of group 1 are read while the
  // MFMAs of group 0 run
  auto compute = [&](int kstep) {
    const unsigned char *sA = smem + (kstep % NS) * STAGE;
    const unsigned char *sB = sA + BM * 64;
    u32x4 af[2][TM], bfg[2][TN];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int b = 0; b < TN; ++b) bfg[g][b] = *(const u32x4 *)(sB + swz64(wn * WTN + b * 32 + l32, g * 2 + half));
#pragma unroll
      for (int a = 0; a < TM; ++a) af[g][a] = *(const u32x4 *)(sA + swz64((a * WM + wm) * 32 + l32, g * 2 + half));
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) Mma<bf16>::run(&bfg[g][b], &af[g][a], acc[a][b]);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // reads of group 0
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // MFMAs of group 0 with the reads of group 1
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // group 1
  };

  while (true) {
    const TileI cur = decode_tile<bf16, BM, false>(p, lt, nk);
    set_src(cur);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nk) issue(s);
    // the first step's loads are the oldest: all but those issued after them
    if (nk >= 3) close_step(IC<8 * (NS - 2)>{});
    else if (nk == 2) close_step(IC<8>{});
    else close_step(IC<0>{});
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;
    int kt = 0;
    for (; kt + NS - 1 < nk; ++kt) {  // steady state: NS - 1 steps in flight
      issue(kt + NS - 1);
      compute(kt);
      close_step(IC<8 * (NS - 2)>{});
    }
    for (; kt < nk; ++kt) {  // drain: steps kt + 1 .. nk - 1 are in flight
      compute(kt);
      if (kt + 2 < nk) close_step(IC<8>{});  // NS == 4: at most kt + 2 issued after kt + 1
      else close_step(IC<0>{});
    }
    store_tile<TO, EPI, BN, WTN, WM, TM, TN>(p, acc, cur.m0, cur.rows, cur.nt, 0, wm, wn, half, l32, nullptr);
    lt += per;
    if (lt >= lt_end) break;
  }
}

}  // namespace lmoe
