// Tiled MFMA GEMM for M > 16 rows (batched drafter blocks, verification of a batch, long
// injections): acc[m][n] = sum_k A[m][k] W[n][k] with optional A-side RMSNorm and a fused
// epilogue (epilogue.h).  Operand layouts as in the GEMV: W (bf16) in B-fragment order,
// float32 activations in A-fragment order, caller-supplied bf16 rows (the tapped features
// of the fusion GEMM) row-major.
#include "gemm_common.h"

namespace dflash {

// ---------------------------------------------------------------------------------------
// M > 16: WGM x WGN waves, each wave TM x TN MFMA tiles (16 x 16), so a workgroup covers
// (16 TM WGM) x (16 TN WGN) outputs.  An LDS stage holds KSUB MFMA k-steps (BK = 32 KSUB),
// double-buffered; DEPTH stages of global loads are in flight in registers while one is
// computed (the loads are unconditional, the stage index clamped, so the compiler counts
// them and never drains the ring).  LDS holds the operands in fragment order - A as (hi,
// lo) bf16 pairs split from the float32 activations on the way in, W as it is stored - so
// every MFMA operand read is one contiguous, conflict-free 1 KB per wave.  Grid: tiles
// M-fastest, remapped so the M tiles of one W column block run on one XCD (one L2).
template <typename TA, int WGM, int WGN, int TM, int TN, int KSUB, int DEPTH, bool NORM, int KIND>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_mfma_bf16(GemmArgs ga) {
  constexpr bool TWO = AIsFloat<TA>::value;
  constexpr int NT_ = 64 * WGM * WGN;             // threads
  constexpr int BM = 16 * TM * WGM, BN = 16 * TN * WGN;   // workgroup tile
  constexpr int RB = BM / 16, NB = BN / 16;       // 16-row A blocks, 16-column W tiles
  constexpr int NP = TWO ? 2 : 1;                 // A planes in LDS: hi (, lo)
  // staging slots per thread and k-step: A float32: RB x 2 halves x 64 lanes float4;
  // A bf16 (row-major rows): RB x 64 lanes x 16 B; W: NB x 64 lanes x 16 B
  constexpr int AS = TWO ? RB * 2 * 64 / NT_ : RB * 64 / NT_;
  constexpr int WS = NB * 64 / NT_;
  static_assert(AS >= 1 && WS >= 1 && AS * NT_ == (TWO ? RB * 128 : RB * 64) && WS * NT_ == NB * 64,
                "tile does not split evenly over the threads");
  static_assert(DEPTH == 2 || DEPTH == 3, "ring depth");
  __shared__ __attribute__((aligned(16))) bf16x8 As[2][NP][KSUB][RB][64];
  __shared__ __attribute__((aligned(16))) bf16x8 Ws[2][KSUB][NB][64];
  __shared__ float ss_part[NORM ? BM : 1][NORM ? 9 : 1];
  __shared__ float rstd_s[NORM ? BM : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = w / WGN, wn = w % WGN;
  const int M = ga.M, N = ga.N, K = ga.K, KS = K >> 5;
  const int NST = KS / KSUB;                      // stages (K % (32 KSUB) == 0)
  const int MB = (M + 15) >> 4, NT = (N + 15) >> 4;
  const int mt_n = (M + BM - 1) / BM, nt_n = (N + BN - 1) / BN;
  const int T = mt_n * nt_n;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int m0 = (t % mt_n) * BM, n0 = (t / mt_n) * BN;

  // ---- staging slots ----
  const TA* ap[AS];
  int a_rb[AS], a_lane[AS], a_h[AS];
#pragma unroll
  for (int j = 0; j < AS; ++j) {
    const int q = tid + NT_ * j;
    if constexpr (TWO) {
      a_rb[j] = q >> 7;
      a_h[j] = (q >> 6) & 1;
      a_lane[j] = q & 63;
      const int mb = min((m0 >> 4) + a_rb[j], MB - 1);
      ap[j] = (const TA*)ga.A + ((size_t)mb * KS * 2 + a_h[j]) * 256 + a_lane[j] * 4;
    } else {
      a_rb[j] = q >> 6;
      a_h[j] = 0;
      a_lane[j] = q & 63;
      const int row = min(m0 + a_rb[j] * 16 + (a_lane[j] & 15), M - 1);
      ap[j] = (const TA*)ga.A + (size_t)row * ga.lda + (a_lane[j] >> 4) * 8;
    }
  }
  const bf16* wp[WS];
  int w_nt[WS], w_lane[WS];
#pragma unroll
  for (int j = 0; j < WS; ++j) {
    const int q = tid + NT_ * j;
    w_nt[j] = q >> 6;
    w_lane[j] = q & 63;
    wp[j] = wblock(ga.B, min((n0 >> 4) + w_nt[j], NT - 1), 0, KS) + w_lane[j] * 8;
  }
  const bf16* gk = NORM ? (const bf16*)ga.norm_g : nullptr;
  float ss[AS];
#pragma unroll
  for (int j = 0; j < AS; ++j) ss[j] = 0.f;

  // a stage's activations, their RMSNorm gains and its weights, loaded together (a gain
  // loaded only when the stage is copied to LDS would be waited for at once and drain the
  // load ring)
  struct Stage {
    float ra[KSUB][AS][TWO ? 4 : 8];
    bf16x4 rg[NORM ? KSUB : 1][NORM ? AS : 1];
    bf16x8 rw[KSUB][WS];
  };
  Stage s0, s1, s2;
  auto gload = [&](Stage& st, int stage) {
#pragma unroll
    for (int u = 0; u < KSUB; ++u) {
      const int ks = stage * KSUB + u;
#pragma unroll
      for (int j = 0; j < AS; ++j) {
        if constexpr (TWO) {
          const float4 x = *(const float4*)(ap[j] + (size_t)ks * 512);
          st.ra[u][j][0] = x.x; st.ra[u][j][1] = x.y; st.ra[u][j][2] = x.z; st.ra[u][j][3] = x.w;
          if constexpr (NORM)
            st.rg[u][j] = *(const bf16x4*)(gk + ks * 32 + 8 * (a_lane[j] >> 4) + 4 * a_h[j]);
        } else {
          load8(ap[j] + (size_t)ks * 32, st.ra[u][j]);
        }
      }
#pragma unroll
      for (int j = 0; j < WS; ++j) st.rw[u][j] = *(const bf16x8*)(wp[j] + (size_t)ks * 512);
    }
  };
  // staged stage -> LDS buffer `buf` (RMSNorm statistics and gain on the way)
  auto lstore = [&](Stage& st, int buf, int stage) {
#pragma unroll
    for (int u = 0; u < KSUB; ++u) {
#pragma unroll
      for (int j = 0; j < AS; ++j) {
        if constexpr (AIsPair<TA>::value) {
          As[buf][a_h[j]][u][a_rb[j]][a_lane[j]] = *(const bf16x8*)&st.ra[u][j][0];
        } else if constexpr (TWO) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = st.ra[u][j][e];
            if constexpr (NORM) {
              ss[j] += x * x;
              x *= (float)st.rg[u][j][e];
            }
            v[e] = x;
            v[4 + e] = 0.f;
          }
          bf16x8 hi, lo;
          split8(v, hi, lo);
          bf16x4* dh = (bf16x4*)&As[buf][0][u][a_rb[j]][a_lane[j]] + a_h[j];
          bf16x4* dl = (bf16x4*)&As[buf][NP - 1][u][a_rb[j]][a_lane[j]] + a_h[j];
          *dh = bf16x4{hi[0], hi[1], hi[2], hi[3]};
          *dl = bf16x4{lo[0], lo[1], lo[2], lo[3]};
        } else {
          bf16x8 hi, lo;
          split8(st.ra[u][j], hi, lo);
          As[buf][0][u][a_rb[j]][a_lane[j]] = hi;
        }
      }
#pragma unroll
      for (int j = 0; j < WS; ++j) Ws[buf][u][w_nt[j]][w_lane[j]] = st.rw[u][j];
    }
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KSUB; ++u) {
      bf16x8 wf[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) wf[j] = Ws[buf][u][wn * TN + j][lane];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const bf16x8 af = As[buf][p][u][wm * TM + i][lane];
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  };
  // ring: stage q is computed from LDS buffer q % 2 while the next DEPTH stages are in
  // flight; then stage q+1 moves to the other buffer.  Past the last stage the loads still
  // run (clamped, harmless) so that every slot issues the same instructions.
  const int last = NST - 1;
  gload(s0, 0);
  gload(s1, min(1, last));
  if constexpr (DEPTH == 3) gload(s2, min(2, last));
  lstore(s0, 0, 0);
  __syncthreads();
  auto body = [&](int q, Stage& ld, Stage& nx) {
    gload(ld, min(q + DEPTH, last));
    if (q < NST) compute(q & 1);
    if (q + 1 < NST) lstore(nx, (q + 1) & 1, q + 1);
    __syncthreads();
  };
  if constexpr (DEPTH == 3) {
    for (int q = 0; q < NST; q += 3) {
      body(q, s0, s1);
      body(q + 1, s1, s2);
      body(q + 2, s2, s0);
    }
  } else {
    for (int q = 0; q < NST; q += 2) {
      body(q, s0, s1);
      body(q + 1, s1, s0);
    }
  }
  if (NORM) {
    // row rb*16 + (lane & 15) collects its 8 contributors (lane >> 4, half) in a fixed order
#pragma unroll
    for (int j = 0; j < AS; ++j) ss_part[a_rb[j] * 16 + (a_lane[j] & 15)][(a_lane[j] >> 4) * 2 + a_h[j]] = ss[j];
    __syncthreads();
    if (tid < BM) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += ss_part[tid][i];
      rstd_s[tid] = 1.0f / sqrtf(s / (float)K + ga.eps);
    }
    __syncthreads();
  }
  unsigned long long best[TM][4];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) best[i][e] = 0ull;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int lr0 = (wm * TM + i) * 16 + g * 4;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = NORM ? acc[i][j][e] * rstd_s[lr0 + e] : acc[i][j][e];
      tile_epilogue<bf16, KIND>(ga, m0 + lr0, n0 + (wn * TN + j) * 16 + r, v, r, best[i]);
    }
  if (KIND == EPI_ARGMAX && r == 0) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + (wm * TM + i) * 16 + g * 4 + e;
        if (row < M && best[i][e]) atomicMax(&ga.e.keys[row], best[i][e]);
      }
  }
}

// ---------------------------------------------------------------------------------------
// M > 16 with the weights going straight to registers.  4 waves; wave w owns the TN 16-column
// tiles n0/16 + w TN + j (j < TN) of the workgroup's BN = 64 TN columns for all BM rows, so
// every weight fragment is loaded from HBM by exactly one wave, into its registers, and used
// there: no LDS traffic for W.  The BM activation rows are shared by the 4 waves through a
// double-buffered LDS stage of KSUB k-steps (fragment order; float32 rows split into (hi,
// lo) bf16 pairs on the way in, RMSNorm statistics gathered there).  Per k-step a wave reads
// BM/16 A fragments (per plane) from LDS and issues TN MFMAs on each, so LDS reads take
// 1/TN of the MFMA time.  Weights run three stages ahead in a register ring (two at TN = 8,
// whose 128 accumulators leave room for no more at two waves per SIMD), the activations one
// stage ahead.  Grid: tiles M-fastest, rounded up to a multiple of 8 and remapped so each
// XCD gets a contiguous range: the row tiles of one weight column block run on one XCD
// (their repeated weight reads hit that XCD's L2).
template <typename TA, int BM, int TN, int KSUB, bool NORM, int KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TN >= 8 ? 2 : 1, 8)))
void gemm_wdirect_bf16(GemmArgs ga) {
  constexpr bool TWO = AIsFloat<TA>::value;
  constexpr int NT_ = 256;
  constexpr int RB = BM / 16, BN = 64 * TN;
  constexpr int NP = TWO ? 2 : 1;
  // activation staging slots per thread and k-step: float32: RB x 2 halves x 64 lanes of
  // float4; bf16 (row-major rows): RB x 64 lanes x 16 B
  constexpr int AS = TWO ? RB * 2 * 64 / NT_ : RB * 64 / NT_;
  static_assert(AS >= 1 && AS * NT_ == (TWO ? RB * 128 : RB * 64), "row tile does not split over the threads");
  
  // epilogue chunk: EPC row blocks of accumulators per wave go through LDS at a time (two at
  // TN = 8, so that two workgroups' LDS fit one CU)
  constexpr int EPC = TN >= 8 ? 2 : (RB * TN * 4 <= 128 ? RB : RB / 2);
  constexpr int AS_BYTES = 2 * NP * KSUB * RB * 1024, EP_BYTES = 4 * EPC * TN * 1024;
  __shared__ __attribute__((aligned(16))) char smem[AS_BYTES > EP_BYTES ? AS_BYTES : EP_BYTES];
  bf16x8 (*As)[NP][KSUB][RB][64] = (bf16x8 (*)[NP][KSUB][RB][64])smem;
  __shared__ float ss_part[NORM ? BM : 1][NORM ? 9 : 1];
  __shared__ float rstd_s[NORM ? BM : 1];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int M = ga.M, N = ga.N, K = ga.K, KS = K >> 5;
  const int NST = KS / KSUB;                      // K % (32 KSUB) == 0 (checked by the launcher)
  const int MB = (M + 15) >> 4, NTl = (N + 15) >> 4;
  const int mt_n = (M + BM - 1) / BM, nt_n = (N + BN - 1) / BN;
  const int T = mt_n * nt_n;
  const int G = gridDim.x;
  int t = blockIdx.x;
  if ((G & 7) == 0) t = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  if (t >= T) return;
  const int m0 = (t % mt_n) * BM, n0 = (t / mt_n) * BN;

  // ---- activation staging slots ----
  const TA* ap[AS];
  int a_rb[AS], a_lane[AS], a_h[AS];
#pragma unroll
  for (int j = 0; j < AS; ++j) {
    const int q = tid + NT_ * j;
    if constexpr (TWO) {
      a_rb[j] = q >> 7;
      a_h[j] = (q >> 6) & 1;
      a_lane[j] = q & 63;
      const int mb = min((m0 >> 4) + a_rb[j], MB - 1);
      ap[j] = (const TA*)ga.A + ((size_t)mb * KS * 2 + a_h[j]) * 256 + a_lane[j] * 4;
    } else {
      a_rb[j] = q >> 6;
      a_h[j] = 0;
      a_lane[j] = q & 63;
      const int row = min(m0 + a_rb[j] * 16 + (a_lane[j] & 15), M - 1);
      ap[j] = (const TA*)ga.A + (size_t)row * ga.lda + (a_lane[j] >> 4) * 8;
    }
  }
  // ---- this wave's weight tiles (clamped: columns past N are computed and discarded) ----
  const bf16* wp[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j)
    wp[j] = wblock(ga.B, min((n0 >> 4) + w * TN + j, NTl - 1), 0, KS) + lane * 8;
  const bf16* gk = NORM ? (const bf16*)ga.norm_g : nullptr;
  float ss[AS];
#pragma unroll
  for (int j = 0; j < AS; ++j) ss[j] = 0.f;

  // activations of a stage with their RMSNorm gains, loaded together one body ahead of
  // their copy to LDS (a load waited for right after it is issued would drain the weight
  // ring)
  struct AStage {
    float ra[KSUB][AS][TWO ? 4 : 8];
    bf16x4 rg[NORM ? KSUB : 1][NORM ? AS : 1];
  };
  auto gload_a = [&](AStage& sa, int stage) {
    auto& ra = sa.ra;
    auto& rg = sa.rg;
#pragma unroll
    for (int u = 0; u < KSUB; ++u) {
      const int ks = stage * KSUB + u;
#pragma unroll
      for (int j = 0; j < AS; ++j) {
        if constexpr (TWO) {
          const float4 x = *(const float4*)(ap[j] + (size_t)ks * 512);
          ra[u][j][0] = x.x; ra[u][j][1] = x.y; ra[u][j][2] = x.z; ra[u][j][3] = x.w;
          if constexpr (NORM)
            rg[u][j] = *(const bf16x4*)(gk + ks * 32 + 8 * (a_lane[j] >> 4) + 4 * a_h[j]);
        } else {
          load8(ap[j] + (size_t)ks * 32, ra[u][j]);
        }
      }
    }
  };
  // staged activations of `stage` -> LDS buffer `buf` (RMSNorm statistics and gain on the
  // way; a clamped repeat of the last stage is stored but not counted)
  auto lstore_a = [&](const AStage& sa, int buf, int stage, bool count) {
    const auto& ra = sa.ra;
    const auto& rg = sa.rg;
#pragma unroll
    for (int u = 0; u < KSUB; ++u) {
#pragma unroll
      for (int j = 0; j < AS; ++j) {
        if constexpr (AIsPair<TA>::value) {
          // this slot's 16 bytes are plane a_h of its lane: copied as they are
          As[buf][a_h[j]][u][a_rb[j]][a_lane[j]] = *(const bf16x8*)&ra[u][j][0];
        } else if constexpr (TWO) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = ra[u][j][e];
            if constexpr (NORM) {
              ss[j] += count ? x * x : 0.f;
              x *= (float)rg[u][j][e];
            }
            v[e] = x;
            v[4 + e] = 0.f;
          }
          bf16x8 hi, lo;
          split8(v, hi, lo);
          bf16x4* dh = (bf16x4*)&As[buf][0][u][a_rb[j]][a_lane[j]] + a_h[j];
          bf16x4* dl = (bf16x4*)&As[buf][NP - 1][u][a_rb[j]][a_lane[j]] + a_h[j];
          *dh = bf16x4{hi[0], hi[1], hi[2], hi[3]};
          *dl = bf16x4{lo[0], lo[1], lo[2], lo[3]};
        } else {
          bf16x8 hi, lo;
          split8(ra[u][j], hi, lo);
          As[buf][0][u][a_rb[j]][a_lane[j]] = hi;
        }
      }
    }
  };
  typedef bf16x8 WStage[KSUB][TN];
  auto gload_w = [&](WStage& wr, int stage) {
#pragma unroll
    for (int u = 0; u < KSUB; ++u)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        wr[u][j] = *(const bf16x8*)(wp[j] + (size_t)(stage * KSUB + u) * 512);
  };

  f32x4 acc[RB][TN];
#pragma unroll
  for (int i = 0; i < RB; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // the RB fragments of the next (k-step, plane) group are read from LDS while the MFMAs of
  // the current group issue, so one wave per SIMD does not wait on LDS latency
  auto compute = [&](int buf, const WStage& wr) {
    constexpr int NG = KSUB * NP;
    bf16x8 fa[2][RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) fa[0][i] = As[buf][0][0][i][lane];
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      const int u = q / NP;
      if (q + 1 < NG) {
#pragma unroll
        for (int i = 0; i < RB; ++i) fa[(q + 1) & 1][i] = As[buf][(q + 1) % NP][(q + 1) / NP][i][lane];
      }
#pragma unroll
      for (int i = 0; i < RB; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[q & 1][i], wr[u][j], acc[i][j], 0, 0, 0);
    }
  };

  // ring: stage q is computed with its weights from ring slot q % WDEPTH and its
  // activations from LDS buffer q % 2; then the activations of stage q + 1 (loaded one body
  // earlier) go to the other buffer, and the freed slots reload stage q + 2 (activations)
  // and q + WDEPTH (weights).  Loads past the last stage are clamped to it (L2 hits), so every body issues
  // the same instructions and the compiler keeps the ring in flight.  (A deeper ring - four
  // weight stages, two activation stages - measured slower: it leaves the compiler too few
  // registers to schedule the MFMAs.)
  const int last = NST - 1;
  constexpr int WDEPTH = TN >= 8 ? 2 : 3;
  WStage w0, w1, w2;
  AStage an;
  gload_w(w0, 0);
  gload_w(w1, min(1, last));
  if constexpr (WDEPTH == 3) gload_w(w2, min(2, last));
  gload_a(an, 0);
  lstore_a(an, 0, 0, true);
  gload_a(an, min(1, last));
  __syncthreads();
  auto body = [&](int q, WStage& wr) {
    if (q < NST) compute(q & 1, wr);
    lstore_a(an, (q + 1) & 1, min(q + 1, last), q + 1 < NST);
    gload_a(an, min(q + 2, last));
    gload_w(wr, min(q + WDEPTH, last));
    __syncthreads();
  };
  if constexpr (WDEPTH == 3) {
    for (int q = 0; q < NST; q += 3) {
      body(q, w0);
      body(q + 1, w1);
      body(q + 2, w2);
    }
  } else {
    for (int q = 0; q < NST; q += 2) {
      body(q, w0);
      body(q + 1, w1);
    }
  }
  if (NORM) {
    // row rb*16 + (lane & 15) collects its 8 contributors (lane >> 4, half) in a fixed order
#pragma unroll
    for (int j = 0; j < AS; ++j) ss_part[a_rb[j] * 16 + (a_lane[j] & 15)][(a_lane[j] >> 4) * 2 + a_h[j]] = ss[j];
    __syncthreads();
    if (tid < BM) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += ss_part[tid][i];
      rstd_s[tid] = 1.0f / sqrtf(s / (float)K + ga.eps);
    }
    __syncthreads();
  }
  // Epilogue: the accumulators of EPC row blocks at a time go to this wave's LDS region and
  // a runtime loop walks them, so the accumulator array is only ever indexed statically
  // (the epilogue code is too large to unroll RB x TN times).
  f32x4* ep = (f32x4*)smem + (size_t)w * EPC * TN * 64;
#pragma unroll
  for (int c = 0; c < RB / EPC; ++c) {
    __syncthreads();   // LDS stage buffers / previous chunk no longer read
#pragma unroll
    for (int i = 0; i < EPC; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) ep[(i * TN + j) * 64 + lane] = acc[c * EPC + i][j];
    __syncthreads();
#pragma unroll 1
    for (int i = 0; i < EPC; ++i) {
      const int lr0 = (c * EPC + i) * 16 + g * 4;
      unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const f32x4 a = ep[(i * TN + j) * 64 + lane];
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = NORM ? a[e] * rstd_s[lr0 + e] : a[e];
        tile_epilogue<bf16, KIND>(ga, m0 + lr0, n0 + (w * TN + j) * 16 + r, v, r, best);
      }
      if (KIND == EPI_ARGMAX && r == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + lr0 + e;
          if (row < M && best[e]) atomicMax(&ga.e.keys[row], best[e]);
        }
      }
    }
  }
}

struct MfmaLaunch {
  template <typename TA, bool NORM, int KIND>
  static hipError_t run(const GemmArgs& ga, hipStream_t st) {
    const int M = ga.M, N = ga.N;
    auto wgs = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    const int ks = ga.K >> 5;
#define WD_LAUNCH(BM, TN)                                                                     \
  return launch1(gemm_wdirect_bf16<TA, BM, TN, 2, NORM, KIND>, dim3((wgs(BM, 64 * TN) + 7) / 8 * 8), \
                 dim3(256), st, ga)
#define WD_LAUNCH1(BM, TN)                                                                    \
  return launch1(gemm_wdirect_bf16<TA, BM, TN, 1, NORM, KIND>, dim3((wgs(BM, 64 * TN) + 7) / 8 * 8), \
                 dim3(256), st, ga)
#define MFMA_LAUNCH(WGM, WGN, TM, TN, KSUB, DEPTH)                                             \
  return launch1(gemm_mfma_bf16<TA, WGM, WGN, TM, TN, KSUB, DEPTH, NORM, KIND>,               \
                 dim3(wgs(16 * TM * WGM, 16 * TN * WGN)), dim3(64 * WGM * WGN), st, ga)
    // Choice measured on the Qwen3-8B shapes at M = 256 and the 512-row injection: when
    // 64 x 128 tiles give every CU work (gate/up, LM head, injection K/V, the fusion GEMM over
    // 512 feature rows), the weight-direct kernel, with 4 weight tiles per wave once there
    // are two workgroups per CU of them; otherwise (QKV, O, down) 64 x 64 LDS-staged tiles,
    // which keep the most CUs busy.  (A stage of two k-steps needs K % 64 == 0 - the
    // weight-direct kernel K % 128 == 0 - else one k-step per stage.)
    if (ks % 4 == 0) {
      if (wgs(64, 128) >= num_cus()) {
        // two workgroups are resident per CU: 64 x 192 tiles when their grid fills whole
        // rounds of those slots clearly better (gate/up at 256 rows: 512 workgroups in one
        // round instead of 768 in one and a half)
        const int slots = 2 * num_cus();
        auto fill = [&](int tn) {
          const int n = wgs(64, 64 * tn);
          return (double)n / ((double)((n + slots - 1) / slots) * slots);
        };
        // operand planes over a wide N (the LM head at 256 rows): 64 x 512 tiles, one k-step
        // per stage, halve the LDS reads and the activation re-reads per MFMA (LM head
        // 655 -> 584 us)
        if constexpr (AIsPair<TA>::value) {
          if (wgs(64, 512) >= 4 * num_cus()) WD_LAUNCH1(64, 8);
        }
        const int tn = wgs(64, 256) >= slots ? 4 : 2;
        if constexpr (AIsFloat<TA>::value) {
          if (wgs(64, 192) >= num_cus() && fill(3) > fill(tn) + 0.1) WD_LAUNCH(64, 3);
        }
        if (tn == 4) WD_LAUNCH(64, 4);
        WD_LAUNCH(64, 2);
      }
      // (32 x 64 tiles when 64 x 64 ones would leave CUs idle, e.g. O and down at 128 rows;
      // bf16 rows - the fusion GEMM over the tapped features - as two-wave workgroups, whose
      // 128 threads split that tile's staging evenly)
      if (wgs(64, 64) < num_cus()) {
        if constexpr (AIsFloat<TA>::value) MFMA_LAUNCH(2, 2, 1, 2, 2, 3);
        else MFMA_LAUNCH(1, 2, 2, 2, 2, 3);
      }
      MFMA_LAUNCH(2, 2, 2, 2, 2, 3);
    }
    if (ks % 2) MFMA_LAUNCH(2, 2, 2, 2, 1, 3);
    MFMA_LAUNCH(2, 2, 2, 2, 2, 3);
#undef MFMA_LAUNCH
#undef WD_LAUNCH
#undef WD_LAUNCH1
  }
};

// bf16 models, K a multiple of 32
hipError_t launch_gemm_mfma(const GemmArgs& ga, hipStream_t st) { return dispatch_gemm<MfmaLaunch>(ga, st); }

}  // namespace dflash
