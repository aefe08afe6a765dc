// Row-resident MFMA GEMM for M > 16 rows (batched drafter blocks, verification of a batch,
// long injections): acc[m][n] = sum_k A[m][k] W[n][k], optional A-side RMSNorm, fused
// epilogue (epilogue.h).  Operands as everywhere in the library: W (bf16) in B-fragment
// order, float32 activations in A-fragment order (taken as compensated (hi, lo) bf16 pairs),
// or caller bf16 rows (the tapped features of the fusion GEMM) row-major.
//
// Shape of the work: M is a few hundred rows and the weights are the bulk of the bytes, so
// a workgroup keeps up to 256 rows - every row of a batch-16 block - and streams its
// 128-column slice of W exactly once.  4 waves, one per SIMD; wave w owns rows
// m0 + 16 TM w .. + 16 TM and all TN = 8 column tiles of the workgroup (TM x TN 16 x 16
// accumulators).  A wave's A rows belong to it alone, so they go from global memory (L2
// mostly: every column workgroup reads the same rows) straight into its registers and are
// converted there (norm gain, sum of squares, hi/lo split): no LDS traffic for A.  The W
// fragments are shared by the 4 waves through a double-buffered LDS stage.  Stages of
// KSUB = 2 k-steps (64 k) run through a 3-deep register ring: the loads of stage q + 3 go
// out as soon as stage q has been computed, so two stages of A and W stay in flight.  All
// loads are unconditional (stage indices clamped), so the compiler counts them and never
// drains the ring at a barrier.
//
// Few column tiles (QKV, O, down, the fusion GEMM): the K range is split over S
// workgroups, which write raw partial accumulators (and partial sums of squares) in
// fragment order; gemm_rows_reduce sums the splits in a fixed order and runs the epilogue,
// so results do not depend on timing.  The (split, tile) work items are numbered
// split-major and each XCD takes a contiguous range of them, so an XCD reads the A rows of
// one or two K ranges only (all splits on every XCD would pull the whole of A from HBM
// into each of the 8 L2s: 8 x 4 MB for 256 float32 rows of K = 4096, as much as the O
// weights).
#include "gemm_common.h"

namespace dflash {

#define ROWS_KSUB 2

// the tile-parallel kernels of gemm_mfma.hip
hipError_t launch_gemm_mfma(const GemmArgs& ga, hipStream_t st);

int rows_splits(const GemmArgs& ga, int tiles);

DF_DEV int xcd_tile(int bid, int T) {
  // consecutive workgroups land on different XCDs (round robin): give each XCD a contiguous
  // range of tiles, so tiles that share operands share an L2
  return (T & 7) == 0 ? (bid & 7) * (T >> 3) + (bid >> 3) : bid;
}

// launch grid of `items` work items: a multiple of 8 (the workgroups past the items exit
// at once), so that xcd_tile always hands out contiguous ranges
static inline int rows_grid(int items) { return (items + 7) / 8 * 8; }

template <typename TA, int NW, int TM, int TN, int DEPTH, bool NORM, int KIND, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 1) void gemm_rows_bf16(GemmArgs ga, SplitArgs sp) {
  constexpr bool TWO = AIsFloat<TA>::value;
  constexpr int KSUB = ROWS_KSUB, NT_ = NW * 64;
  constexpr int BM = NW * 16 * TM, BN = 16 * TN;
  constexpr int WPT = TN * KSUB * 64 / NT_;   // 16-byte W pieces per thread and stage
  constexpr int AV = TWO ? 2 : 1;              // 16-byte A loads per row block and k-step
  static_assert(WPT >= 1 && WPT * NT_ == TN * KSUB * 64, "W stage does not split over the threads");
  static_assert(DEPTH == 2 || DEPTH == 3, "ring depth");
  __shared__ __attribute__((aligned(16))) bf16x8 Ws[2][KSUB][TN][64];
  __shared__ __attribute__((aligned(16))) bf16x8 gsh[NORM ? ROWS_MAX_NORM_K / 8 : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int M = ga.M, N = ga.N, K = ga.K, KS = K >> 5;
  const int MB = (M + 15) >> 4, NT = (N + 15) >> 4;
  const int mt_n = (M + BM - 1) / BM, nt_n = (N + BN - 1) / BN;
  const int T = mt_n * nt_n, S = SPLIT ? sp.splits : 1;
  const int q = xcd_tile(blockIdx.x, gridDim.x);
  if (q >= T * S) return;   // grid padding (whole workgroup, before any barrier)
  const int s = q / T, t = q % T;
  const int m0 = (t % mt_n) * BM, n0 = (t / mt_n) * BN;
  // this split's stages (KS % KSUB == 0, checked by the launcher)
  const int NST_ALL = KS / KSUB;
  const int st0 = (int)((long)NST_ALL * s / S), st1 = (int)((long)NST_ALL * (s + 1) / S);
  const int nst = st1 - st0;
  const int last = st1 - 1;

  // ---- A: this wave's TM row blocks (clamped past M: computed and discarded) ----
  const TA* ap[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int mb = min((m0 >> 4) + w * TM + i, MB - 1);
    if constexpr (TWO)
      ap[i] = (const TA*)ga.A + (size_t)mb * KS * 512 + lane * 4;
    else
      ap[i] = (const TA*)ga.A + (size_t)min(mb * 16 + r, M - 1) * ga.lda + g * 8;
  }
  // ---- W: the pieces this thread stages (fragment f = piece >> 6: k-step f / TN, tile f % TN)
  const bf16* wp[WPT];
  int w_u[WPT], w_t[WPT], w_l[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const int q = tid + NT_ * j;
    const int f = q >> 6;
    w_u[j] = f / TN;
    w_t[j] = f % TN;
    w_l[j] = q & 63;
    wp[j] = wblock(ga.B, min((n0 >> 4) + w_t[j], NT - 1), 0, KS) + w_l[j] * 8;
  }

  struct Stage {
    uint4 a[KSUB][TM][AV];
    bf16x8 wv[WPT];
  };
  auto gload = [&](Stage& st, int stage) {
#pragma unroll
    for (int u = 0; u < KSUB; ++u) {
      const int ks = stage * KSUB + u;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        if constexpr (TWO) {
          st.a[u][i][0] = *(const uint4*)(ap[i] + (size_t)ks * 512);
          st.a[u][i][1] = *(const uint4*)(ap[i] + (size_t)ks * 512 + 256);
        } else {
          st.a[u][i][0] = *(const uint4*)(ap[i] + (size_t)ks * 32);
        }
      }
    }
    // bf16 rows (the fusion GEMM over tapped features, K = 20480): the weights stream with
    // the non-temporal hint (134 -> 123 us at 512 rows); with float rows it measured slower
    // (the K-split QKV / O / down at 256 rows, 33 -> 37 and 39 -> 42 us)
#pragma unroll
    for (int j = 0; j < WPT; ++j) {
      const bf16* p = wp[j] + (size_t)(stage * KSUB + w_u[j]) * 512;
      st.wv[j] = AIsFloat<TA>::value ? *(const bf16x8*)p : wload(p);
    }
  };
  auto wstore = [&](const Stage& st, int buf) {
#pragma unroll
    for (int j = 0; j < WPT; ++j) Ws[buf][w_u[j]][w_t[j]][w_l[j]] = st.wv[j];
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) ss[i] = 0.f;

  auto compute = [&](int buf, const Stage& st, int stage) {
#pragma unroll
    for (int u = 0; u < KSUB; ++u) {
      bf16x8 wf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) wf[j] = Ws[buf][u][j][lane];
      bf16x8 gv;
      if constexpr (NORM) gv = gsh[(stage * KSUB + u) * 4 + g];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        bf16x8 hi, lo;
        if constexpr (AIsPair<TA>::value) {
          hi = *(const bf16x8*)&st.a[u][i][0];
          lo = *(const bf16x8*)&st.a[u][i][1];
        } else if constexpr (TWO) {
          const float4 x0 = *(const float4*)&st.a[u][i][0], x1 = *(const float4*)&st.a[u][i][1];
          float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
          if constexpr (NORM) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              ss[i] += v[e] * v[e];
              v[e] *= (float)gv[e];
            }
          }
          split8(v, hi, lo);
        } else {
          hi = *(const bf16x8*)&st.a[u][i][0];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, wf[j], acc[i][j], 0, 0, 0);
        if constexpr (TWO) {
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, wf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };

  // prologue: DEPTH stages in flight, the gains of the whole K in LDS, stage 0's W in LDS
  Stage s0, s1, s2;
  gload(s0, st0);
  gload(s1, min(st0 + 1, last));
  if constexpr (DEPTH == 3) gload(s2, min(st0 + 2, last));
  if constexpr (NORM) {
    for (int i = tid; i < K / 8; i += NT_) gsh[i] = *(const bf16x8*)((const bf16*)ga.norm_g + i * 8);
  }
  wstore(s0, 0);
  __syncthreads();
  // body q: compute stage q (A from its ring slot, W from LDS buffer q % 2), move stage
  // q + 1's W into the other buffer, then refill the slot with stage q + DEPTH
  auto body = [&](int q, Stage& cur, const Stage& nxt) {
    if (q < nst) compute(q & 1, cur, st0 + q);
    wstore(nxt, (q + 1) & 1);
    __syncthreads();
    gload(cur, min(st0 + q + DEPTH, last));
  };
  if constexpr (DEPTH == 3) {
    for (int q = 0; q < nst; q += 3) {
      body(q, s0, s1);
      body(q + 1, s1, s2);
      body(q + 2, s2, s0);
    }
  } else {
    for (int q = 0; q < nst; q += 2) {
      body(q, s0, s1);
      body(q + 1, s1, s0);
    }
  }

  // ---- finish: rows are wave-private, so the sums of squares reduce inside the wave ----
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    ss[i] += __shfl_xor(ss[i], 16, 64);
    ss[i] += __shfl_xor(ss[i], 32, 64);
  }
  if constexpr (SPLIT) {
    // raw partials in fragment order: tile (16-row block mb, 16-column tile nb) of split s
    // is 256 floats, lane l holding rows 4g .. 4g+3 of column r
    const int MBp = sp.mb_pad, NTp = sp.nt_pad;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int mb = (m0 >> 4) + w * TM + i;
      if (mb >= MB) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int nb = (n0 >> 4) + j;
        if (nb >= NT) continue;
        *(f32x4*)(sp.part + (((size_t)s * MBp + mb) * NTp + nb) * 256 + lane * 4) = acc[i][j];
      }
      if (NORM && g == 0) sp.ss[(size_t)s * MBp * 16 + mb * 16 + r] = ss[i];
    }
    return;
  }
  float rs[TM][4];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const float rstd = NORM ? 1.0f / sqrtf(ss[i] / (float)K + ga.eps) : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) rs[i][e] = __shfl(rstd, 4 * g + e, 64);
  }
  // Epilogue: TNC accumulator tiles of one row block at a time go through this wave's LDS
  // region and a runtime loop walks them (the accumulator array is only indexed statically)
  constexpr int TNC = (int)sizeof(Ws) / (NW * 1024) < TN ? (int)sizeof(Ws) / (NW * 1024) : TN;
  static_assert(TNC >= 1 && TN % TNC == 0, "epilogue staging");
  __syncthreads();   // W buffers no longer read
  f32x4* ep = (f32x4*)&Ws[0][0][0][0] + (size_t)w * TNC * 64;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    float rsi[4] = {rs[i][0], rs[i][1], rs[i][2], rs[i][3]};
    const int row0 = m0 + (w * TM + i) * 16 + 4 * g;
    unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int c = 0; c < TN / TNC; ++c) {
#pragma unroll
      for (int j = 0; j < TNC; ++j) ep[j * 64 + lane] = acc[i][c * TNC + j];
#pragma unroll 1
      for (int j = 0; j < TNC; ++j) {
        const f32x4 a = ep[j * 64 + lane];
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a[e] * rsi[e];
        tile_epilogue<bf16, KIND>(ga, row0, n0 + (c * TNC + j) * 16 + r, v, r, best);
      }
    }
    if (KIND == EPI_ARGMAX && r == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (row0 + e < M && best[e]) atomicMax(&ga.e.keys[row0 + e], best[e]);
    }
  }
}

// Sum of the K splits in split order, then the epilogue: one wave per 16 x 16 tile.
template <bool NORM, int KIND>
__global__ __launch_bounds__(256) void gemm_rows_reduce(GemmArgs ga, SplitArgs sp) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int MB = (ga.M + 15) >> 4, NT = (ga.N + 15) >> 4;
  const int tile = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tile >= MB * NT) return;
  const int mb = tile / NT, nb = tile % NT;
  const int S = sp.splits, MBp = sp.mb_pad, NTp = sp.nt_pad;
  // every split's partial is loaded at once (index clamped to a valid split, the extra
  // ones not added), so the sum waits for one memory round trip, not S of them; the sum
  // runs in split order
  f32x4 x[ROWS_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < ROWS_MAX_SPLITS; ++s)
    x[s] = *(const f32x4*)(sp.part + (((size_t)min(s, S - 1) * MBp + mb) * NTp + nb) * 256 + lane * 4);
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < ROWS_MAX_SPLITS; ++s)
    if (s < S) a += x[s];
  float v[4] = {a[0], a[1], a[2], a[3]};
  if constexpr (NORM) {
    float sum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < ROWS_MAX_SPLITS; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) sum[e] += s < S ? sp.ss[(size_t)min(s, S - 1) * MBp * 16 + mb * 16 + 4 * g + e] : 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] *= 1.0f / sqrtf(sum[e] / (float)ga.K + ga.eps);
  }
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
  tile_epilogue<bf16, KIND>(ga, mb * 16 + 4 * g, nb * 16 + r, v, r, best);
  if (KIND == EPI_ARGMAX && r == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = mb * 16 + 4 * g + e;
      if (row < ga.M && best[e]) atomicMax(&ga.e.keys[row], best[e]);
    }
  }
}

struct RowsLaunch {
  template <typename TA, bool NORM, int KIND>
  static hipError_t run(const GemmArgs& ga, hipStream_t st) {
    const int M = ga.M, N = ga.N, KS = ga.K >> 5;
    if (KS % ROWS_KSUB || (NORM && ga.K > ROWS_MAX_NORM_K)) return launch_gemm_mfma(ga, st);
    // rows per workgroup: 256 (4 row blocks per wave) unless the rows fit fewer
    const int tm = M > 128 ? 4 : (M > 64 ? 2 : 1);
    const int bm = 64 * tm, bn = 16 * 8;
    const int tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
    const int S = rows_splits(ga, tiles);
    SplitArgs sp = ga.split;
    sp.splits = S;
    sp.mb_pad = (M + 15) / 16;
    sp.nt_pad = (N + 15) / 16;
    auto grid_of = [&](int bm_, int bn_) { return ((M + bm_ - 1) / bm_) * ((N + bn_ - 1) / bn_); };
#define ROWS_K(NWV, TMV, TNV, DV, SPL) gemm_rows_bf16<TA, NWV, TMV, TNV, DV, NORM, KIND, SPL>
// (ROWS_GO launches and does not return: its uses form one if / else chain)
#define ROWS_GO(NWV, TMV, TNV, DV, SPL)                                                          \
  hipLaunchKernelGGL((ROWS_K(NWV, TMV, TNV, DV, SPL)),                                          \
                     dim3(rows_grid(grid_of(NWV * 16 * TMV, 16 * TNV) * (SPL ? S : 1))), dim3(NWV * 64), \
                     0, st, ga, sp)
    if (S == 1) {
      // enough column tiles to fill the chip.  Up to 128 rows: 8 waves of 16 rows x 128
      // columns, all rows in one workgroup; beyond, the tile-parallel kernels of
      // gemm_mfma.hip, whose 64-row tiles keep two workgroups on every CU (measured on the
      // Qwen3-8B shapes at 128 and 256 rows)
      if (M > 128 || !AIsFloat<TA>::value) return launch_gemm_mfma(ga, st);
      // over a vocabulary-wide N (the LM head at 65 - 128 rows): 4 waves of 32 rows, so each
      // W fragment read from LDS feeds four MFMAs instead of two (batch-8 drafting 1675 ->
      // 1596-1612 us, verify + inject + commit 2596-2612 -> 2514-2532 us on one box)
      if (M > 64 && N >= 65536) ROWS_GO(4, 2, 8, 3, false);
      else if (M > 64) ROWS_GO(8, 1, 8, 3, false);
      else ROWS_GO(4, 1, 8, 3, false);
      return hipGetLastError();
    }
    // K splits: float rows (hi/lo conversion in every wave) as 8 waves, two per SIMD, so that
    // one wave's conversion overlaps the other's matrix ops; bf16 rows (the fusion GEMM over
    // tapped features) as 4 waves of 64 rows (measured at 128, 256 and 512 rows)
    if (AIsFloat<TA>::value && tm == 4) ROWS_GO(8, 2, 8, 2, true);
    else if (AIsFloat<TA>::value && tm == 2) ROWS_GO(8, 1, 8, 3, true);
    else if (tm == 4) ROWS_GO(4, 4, 8, 3, true);
    else if (tm == 2) ROWS_GO(4, 2, 8, 3, true);
    else ROWS_GO(4, 1, 8, 3, true);
#undef ROWS_GO
#undef ROWS_K
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int ntiles = ((M + 15) / 16) * ((N + 15) / 16);
    hipLaunchKernelGGL((gemm_rows_reduce<NORM, KIND>), dim3((ntiles + 3) / 4), dim3(256), 0, st, ga, sp);
    return hipGetLastError();
  }
};

// K splits for `tiles` column/row workgroups: enough to give every CU a workgroup when the
// tiles alone leave more than half of them idle, each split at least 4 stages long, and the
// partials within the caller's split scratch.
int rows_splits(const GemmArgs& ga, int tiles) {
  const int cus = num_cus();
  if (tiles * 2 > cus || !ga.split.part) return 1;
  const int KS = ga.K >> 5, nst = KS / ROWS_KSUB;
  int S = cus / tiles;
  if (S > ROWS_MAX_SPLITS) S = ROWS_MAX_SPLITS;
  if (S > nst / 4) S = nst / 4;
  const size_t per = (size_t)((ga.M + 15) / 16) * ((ga.N + 15) / 16) * 256 * 4;
  while (S > 1 && per * S > ga.split.part_bytes) --S;
  return S < 1 ? 1 : S;
}

hipError_t launch_gemm_rows(const GemmArgs& ga, hipStream_t st) { return dispatch_gemm<RowsLaunch>(ga, st); }

size_t rows_split_bytes(int rows, int max_n) {
  const size_t full = (size_t)ROWS_MAX_SPLITS * ((rows + 15) / 16) * 16 * ((max_n + 15) / 16) * 16 * 4;
  return full < ROWS_SPLIT_BYTES ? full : ROWS_SPLIT_BYTES;
}
size_t rows_split_ss_bytes(int rows) { return (size_t)ROWS_MAX_SPLITS * ((rows + 15) / 16) * 16 * 4; }

}  // namespace dflash
