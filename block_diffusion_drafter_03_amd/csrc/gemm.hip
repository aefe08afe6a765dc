// GEMM kernels with fused epilogues: acc[m][n] = sum_k A[m][k] W[n][k] (y = x W^T),
// optional A-side RMSNorm, then one of the epilogues of epilogue.h.
//
// bfloat16 models: W in B-fragment order and float32 activations in A-fragment order
// (common.h), so every operand load of a wave is one contiguous 1 KB burst.  Activations
// enter the MFMAs as compensated (hi, lo) bf16 pairs; caller-supplied bf16 inputs (the
// tapped features of the fusion GEMM) are row-major and enter as they are.
//  * gemm_gemv_bf16   (M <= 16): the weight-streaming shape of a drafter step.  8 waves
//    split K, a workgroup walks 16-column tiles; see the kernel.
//  * gemm_mfma_bf16   (M > 16): 2 x 2 waves of up to 64 x 64 outputs, A (hi, lo) and W staged
//    through LDS in fragment order, the next K step's loads in flight during the MFMAs.
//  * gemm_f32         (float32 models): VALU 64x64 tiles, BK = 16, row-major operands.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l (r = l % 16, g = l / 16) supplies A[r][8g..8g+7]
// and W row r's k-slice 8g..8g+7; the accumulator holds D[4g + i][r], i = 0..3.
#include "epilogue.h"

namespace dflash {

// Row n of a row-major B operand (float32 models), possibly split into equal segments.
template <typename T>
DF_DEV const T* brow(const BSeg& b, int n) {
  const int s = b.nseg > 1 ? n / b.seg_rows : 0;
  return (const T*)pick8(b.ptr, s) + (size_t)(n - s * b.seg_rows) * b.ldb;
}

// 1 KB B-fragment block (16-row tile t, 32-wide step ks) of fragment-ordered weights,
// possibly split into equal row segments (seg_rows a multiple of 16).
DF_DEV const bf16* wblock(const BSeg& b, int t, int ks, int KS) {
  const int tps = b.seg_rows >> 4;
  const int s = b.nseg > 1 ? t / tps : 0;
  return (const bf16*)pick8(b.ptr, s) + ((size_t)(t - s * tps) * KS + ks) * 512;
}

// the 8 A values of lane (r = lane % 16, g = lane / 16) at row block mb, step ks of
// fragment-ordered float32 activations
DF_DEV void afrag_load8(const float* A, int mb, int ks, int KS, int lane, float v[8]) {
  const float* p = A + ((size_t)(mb * KS + ks) * 2) * 256 + lane * 4;
  const float4 x0 = *(const float4*)p, x1 = *(const float4*)(p + 256);
  v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
  v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
}

DF_DEV unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  const unsigned lo = __shfl_xor((unsigned)(v & 0xFFFFFFFFull), mask, 64);
  const unsigned hi = __shfl_xor((unsigned)(v >> 32), mask, 64);
  return ((unsigned long long)hi << 32) | lo;
}
DF_DEV unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }

// debug copy of a logit: rows j == 0 of each skipB-row block (the drafter's anchors) are
// not drafts and are left out
DF_DEV void logit_store(const EpiArgs& e, int row, int col, int N, float v) {
  if (e.skipB) {
    const int j = row % e.skipB;
    if (j == 0) return;
    row = (row / e.skipB) * (e.skipB - 1) + j - 1;
  }
  e.logits[(size_t)row * N + col] = v;
}

// Epilogue of one 16x16 MFMA tile held in the accumulator layout: v[i] = acc[row0+4g+i][col].
// Pair epilogues are taken by even lanes (their odd neighbour holds column col + 1).
template <typename T, int KIND>
DF_DEV void tile_epilogue(const GemmArgs& ga, int row0, int col, const float v[4], int r,
                          unsigned long long best[4]) {
  const EpiArgs& e = ga.e;
  const int M = ga.M, N = ga.N;
  if constexpr (KIND == EPI_ARGMAX) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + i;
      const bool ok = row < M && col < N;
      if (ok && e.logits) logit_store(e, row, col, N, v[i]);
      unsigned long long k = ok ? pack_argmax_key(v[i], col) : 0ull;
      k = umax64(k, shfl_xor_u64(k, 1));
      k = umax64(k, shfl_xor_u64(k, 2));
      k = umax64(k, shfl_xor_u64(k, 4));
      k = umax64(k, shfl_xor_u64(k, 8));
      best[i] = umax64(best[i], k);
    }
  } else if constexpr (epi_is_pair(KIND)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v1 = __shfl_xor(v[i], 1, 64);
      const int row = row0 + i;
      if (!(r & 1) && row < M && col + 1 < N) epi_pair<T, KIND>(e, row, col, v[i], v1);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = row0 + i;
      if (row < M && col < N) epi_elem<T, KIND>(e, row, col, v[i]);
    }
  }
}

// ---------------------------------------------------------------------------------------
// A operand helpers.  TA = float: fragment-ordered activations, taken as a compensated
// (hi, lo) bf16 pair (two MFMAs per W fragment); TA = bf16: caller rows, one MFMA.
template <typename TA> struct AIsFloat { static constexpr bool value = false; };
template <> struct AIsFloat<float> { static constexpr bool value = true; };

// v (8 raw A values) -> operand pair; with NORM, sum of squares of the raw values is added
// to *ss and v is multiplied by the gain slice gp[0..7] first.
template <bool NORM, bool ACC_SS>
DF_DEV void a_operand(float v[8], const bf16* gp, float* ss, bf16x8& hi, bf16x8& lo) {
  if (NORM) {
    const bf16x8 gv = *(const bf16x8*)gp;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (ACC_SS) *ss += v[e] * v[e];
      v[e] *= (float)gv[e];
    }
  }
  split8(v, hi, lo);
}

// M <= 16: NW waves split K, one 32-wide step per MFMA (pair).
//  * ASTAT (many tiles, K <= 4096): one workgroup per CU walks the tiles; each wave keeps
//    its K-slice of the A rows for all of them, already multiplied by the RMSNorm gain and
//    split into (hi, lo) (rstd is applied in the epilogue): hi in registers, lo in LDS
//    (128 KB: the workgroup owns the CU), so the vector memory path carries only W: a wave
//    issues all of its W loads of a tile at once (CH steps, 1 KB each) and the next tile's
//    loads go out right after the MFMAs, in flight across the reduction.
//  * streamed (few tiles, or K > 4096): A and W are loaded together in chunks of CHS
//    steps; no LDS for A, so several workgroups share a CU and every tile is in flight.
// 8 waves of 512 threads leave each wave 256 registers, so the stationary A, a full tile
// of W in flight and the epilogue never spill.
#define GEMV_MAX_TILES 8   // tiles per workgroup whose epilogue is deferred (non-argmax kinds)
#define GEMV_NW 8          // waves per workgroup

template <typename TA, int NW, bool NORM, bool ASTAT, int KIND>
__global__ __launch_bounds__(NW * 64) void gemm_gemv_bf16(GemmArgs ga) {
  constexpr bool TWO = AIsFloat<TA>::value;
  constexpr int CH = 128 / NW;       // stationary steps per wave (K <= 4096)
  constexpr int CHS = 8;             // streamed chunk
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int M = ga.M, N = ga.N, K = ga.K;
  const int KS = K >> 5;
  const int spw = KS / NW;                       // K % (32 NW) == 0
  const int ks0 = w * spw;
  const int n_tiles = (N + 15) >> 4;
  __shared__ f32x4 red[NW][64];
  __shared__ f32x4 done[GEMV_MAX_TILES][64];
  __shared__ float ss_red[NW][16];
  __shared__ float rstd[16];
  __shared__ bf16x8 alo[ASTAT && TWO ? NW : 1][ASTAT && TWO ? CH : 1][64];
  // running argmax keys of wave 0's lanes (kept out of the main loop's registers)
  __shared__ unsigned long long bsh[KIND == EPI_ARGMAX ? 4 : 1][64];
  const bf16* gk = NORM ? (const bf16*)ga.norm_g + g * 8 : nullptr;
  // this lane's 8 A values of step ks (row r)
  auto load_a = [&](int ks, float v[8]) {
    if constexpr (TWO)
      afrag_load8((const float*)ga.A, 0, ks, KS, lane, v);
    else
      load8((const bf16*)ga.A + (size_t)min(r, M - 1) * ga.lda + (size_t)ks * 32 + g * 8, v);
  };
  int nbuf = 0;
  bool first = true;
  if (KIND == EPI_ARGMAX && w == 0)
#pragma unroll
    for (int i = 0; i < (KIND == EPI_ARGMAX ? 4 : 1); ++i) bsh[i][lane] = 0ull;

  bf16x8 ah[ASTAT ? CH : 1];
  // W loads of this workgroup's first tile go out before the A prologue (independent)
  bf16x8 wn[ASTAT ? CH : 1];
  auto load_w = [&](int t) {
#pragma unroll
    for (int s = 0; s < CH; ++s)
      if (s < spw) wn[s] = *(const bf16x8*)(wblock(ga.B, t, ks0 + s, KS) + lane * 8);
  };
  if constexpr (ASTAT) {
    if (blockIdx.x < n_tiles) load_w(blockIdx.x);
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      if (s < spw) {
        float v[8];
        load_a(ks0 + s, v);
        bf16x8 lo;
        a_operand<NORM, true>(v, gk + (size_t)(ks0 + s) * 32, &ss, ah[s], lo);
        if constexpr (TWO) alo[w][s][lane] = lo;
      }
    }
    if (NORM) {
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      if (g == 0) ss_red[w][r] = ss;
      __syncthreads();
      if (threadIdx.x < 16) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += ss_red[ww][threadIdx.x];
        rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)K + ga.eps);
      }
      __syncthreads();
    }
  }

  for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f}, acc2 = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ASTAT) {
#pragma unroll
      for (int s = 0; s < CH; ++s)
        if (s < spw) {
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[s], wn[s], acc, 0, 0, 0);
          if constexpr (TWO) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[w][s][lane], wn[s], acc2, 0, 0, 0);
        }
      // the next tile's W loads are in flight across the barrier and the reduction
      if (t + gridDim.x < n_tiles) load_w(t + gridDim.x);
    } else {
      float ss = 0.f;
      for (int c0 = 0; c0 < spw; c0 += CHS) {
        bf16x8 wf[CHS];
        float av[CHS][8];
#pragma unroll
        for (int s = 0; s < CHS; ++s) {
          const int k = ks0 + min(c0 + s, spw - 1);
          wf[s] = *(const bf16x8*)(wblock(ga.B, t, k, KS) + lane * 8);
          load_a(k, av[s]);
        }
#pragma unroll
        for (int s = 0; s < CHS; ++s)
          if (c0 + s < spw) {
            bf16x8 hi, lo;
            if (first)
              a_operand<NORM, true>(av[s], gk + (size_t)(ks0 + c0 + s) * 32, &ss, hi, lo);
            else
              a_operand<NORM, false>(av[s], gk + (size_t)(ks0 + c0 + s) * 32, &ss, hi, lo);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, wf[s], acc, 0, 0, 0);
            if constexpr (TWO) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, wf[s], acc2, 0, 0, 0);
          }
      }
      if (NORM && first) {
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        if (g == 0) ss_red[w][r] = ss;
      }
    }
    red[w][lane] = acc + acc2;
    __syncthreads();
    if (NORM && !ASTAT && first) {
      if (threadIdx.x < 16) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += ss_red[ww][threadIdx.x];
        rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)K + ga.eps);
      }
      __syncthreads();
    }
    first = false;
    if (w == 0) {
      f32x4 s = red[0][lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) s += red[ww][lane];
      if constexpr (KIND == EPI_ARGMAX) {
        float v[4];
        unsigned long long best[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[i] = NORM ? s[i] * rstd[g * 4 + i] : s[i];
          best[i] = bsh[i][lane];
        }
        tile_epilogue<bf16, KIND>(ga, g * 4, t * 16 + r, v, r, best);
#pragma unroll
        for (int i = 0; i < 4; ++i) bsh[i][lane] = best[i];
      } else {
        done[nbuf][lane] = s;   // epilogue deferred until the A registers are dead
      }
    }
    ++nbuf;
    __syncthreads();
  }
  if constexpr (KIND != EPI_ARGMAX) {
    // every wave takes buffered tiles: the epilogues run in parallel, off the main loop's
    // register budget
    unsigned long long best[4];
    for (int i = w; i < nbuf; i += NW) {
      const f32x4 s = done[i][lane];
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = NORM ? s[e] * rstd[g * 4 + e] : s[e];
      tile_epilogue<bf16, KIND>(ga, g * 4, (blockIdx.x + i * gridDim.x) * 16 + r, v, r, best);
    }
  }
  if (KIND == EPI_ARGMAX && w == 0 && r == 0) {
#pragma unroll
    for (int i = 0; i < (KIND == EPI_ARGMAX ? 4 : 1); ++i) {
      const int row = g * 4 + i;
      const unsigned long long k = bsh[i][lane];
      if (row < M && k) atomicMax(&ga.e.keys[row], k);
    }
  }
}

// Tuning knobs read once from the environment (benchmark sweeps): DFLASH_GEMV=1 forces the
// tiled kernel for M <= 16; DFLASH_GEMV_STREAM_TILES sets the largest tile count that uses
// the streamed-A form (default: one tile per CU).
static int env_knob(const char* name, int dflt) {
  const char* s = getenv(name);
  return s && *s ? atoi(s) : dflt;
}
static int gemv_variant() {
  static const int v = env_knob("DFLASH_GEMV", 0);
  return v;
}
static int num_cus();
static int gemv_stream_tiles() {
  static const int v = env_knob("DFLASH_GEMV_STREAM_TILES", num_cus());
  return v;
}
// DFLASH_GEMM_TILE forces the M > 16 workgroup tile and K staging (see launch_kind)
static int gemm_tile_knob() {
  static const int v = env_knob("DFLASH_GEMM_TILE", 0);
  return v;
}

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

  struct Stage {
    float ra[KSUB][AS][TWO ? 4 : 8];
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
      const int ks = stage * KSUB + u;
#pragma unroll
      for (int j = 0; j < AS; ++j) {
        if constexpr (TWO) {
          float v[8];
          const int k0 = ks * 32 + 8 * (a_lane[j] >> 4) + 4 * a_h[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float x = st.ra[u][j][e];
            if (NORM) {
              ss[j] += x * x;
              x *= (float)gk[k0 + e];
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
template <bool NORM, int KIND>
__global__ __launch_bounds__(256) void gemm_f32(GemmArgs ga) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  __shared__ float rstd_s[64];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int M = ga.M, N = ga.N, K = ga.K;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const float* ap = (const float*)ga.A + (size_t)min(m0 + lr, M - 1) * ga.lda + lk;
  const float* bp = brow<float>(ga.B, min(n0 + lr, N - 1)) + lk;
  const float* gk = NORM ? (const float*)ga.norm_g + lk : nullptr;
  float ss = 0.f;
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float a = ap[k0 + e];
      if (NORM) {
        ss += a * a;
        a *= gk[k0 + e];
      }
      As[lk + e][lr] = a;
      Bs[lk + e][lr] = bp[k0 + e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (NORM) {
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    if ((tid & 3) == 0) rstd_s[lr] = 1.0f / sqrtf(ss / (float)K + ga.eps);
    __syncthreads();
  }
  const EpiArgs& e = ga.e;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    const float sc = NORM ? rstd_s[ty * 4 + i] : 1.f;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = acc[i][j] * sc;
    const int col0 = n0 + tx * 4;
    if constexpr (KIND == EPI_ARGMAX) {
      unsigned long long k = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (row < M && col0 + j < N) {
          if (e.logits) logit_store(e, row, col0 + j, N, v[j]);
          k = umax64(k, pack_argmax_key(v[j], col0 + j));
        }
      k = umax64(k, shfl_xor_u64(k, 1));
      k = umax64(k, shfl_xor_u64(k, 2));
      k = umax64(k, shfl_xor_u64(k, 4));
      k = umax64(k, shfl_xor_u64(k, 8));
      if (tx == 0 && row < M && k) atomicMax(&e.keys[row], k);
    } else if (row < M) {
      if constexpr (epi_is_pair(KIND)) {
#pragma unroll
        for (int j = 0; j < 4; j += 2)
          if (col0 + j + 1 < N) epi_pair<float, KIND>(e, row, col0 + j, v[j], v[j + 1]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (col0 + j < N) epi_elem<float, KIND>(e, row, col0 + j, v[j]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------
static int g_num_cus = 0;
static int num_cus() {
  if (!g_num_cus) {
    int dev = 0;
    hipGetDevice(&dev);
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0)
      g_num_cus = p.multiProcessorCount;
    else
      g_num_cus = 256;
  }
  return g_num_cus;
}

template <typename TA, bool NORM, int KIND>
static hipError_t launch_kind(int dt, const GemmArgs& ga, hipStream_t st) {
  const int M = ga.M, N = ga.N;
  if (dt == F32) {
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL((gemm_f32<NORM, KIND>), grid, dim3(256), 0, st, ga);
    return hipGetLastError();
  }
  const int n_tiles = (N + 15) / 16;
  if (M <= 16 && ga.K % (32 * GEMV_NW) == 0 && gemv_variant() != 1) {
    // few tiles (up to gemv_stream_tiles(), default one per CU) or K > 4096: one workgroup
    // per tile, A streamed with W, so that several workgroups may share a CU and every tile
    // is in flight at once; otherwise one workgroup per CU with the A slice stationary,
    // walking the tiles (the deferred epilogue buffer bounds the tiles per workgroup)
    if (n_tiles <= gemv_stream_tiles() || ga.K > 4096) {
      int grid = n_tiles;
      if (grid > 8 * num_cus()) grid = 8 * num_cus();
      if (KIND != EPI_ARGMAX && grid * GEMV_MAX_TILES < n_tiles)
        grid = (n_tiles + GEMV_MAX_TILES - 1) / GEMV_MAX_TILES;
      hipLaunchKernelGGL((gemm_gemv_bf16<TA, GEMV_NW, NORM, false, KIND>), dim3(grid), dim3(GEMV_NW * 64), 0, st, ga);
    } else {
      int grid = n_tiles < num_cus() ? n_tiles : num_cus();
      if (KIND != EPI_ARGMAX && grid * GEMV_MAX_TILES < n_tiles)
        grid = (n_tiles + GEMV_MAX_TILES - 1) / GEMV_MAX_TILES;
      hipLaunchKernelGGL((gemm_gemv_bf16<TA, GEMV_NW, NORM, true, KIND>), dim3(grid), dim3(GEMV_NW * 64), 0, st, ga);
    }
    return hipGetLastError();
  }
  // the largest workgroup tile that still gives every CU work
  auto wgs = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  const int tile = gemm_tile_knob();
#define MFMA_LAUNCH(WGM, WGN, TM, TN, KSUB, DEPTH)                                             \
  hipLaunchKernelGGL((gemm_mfma_bf16<TA, WGM, WGN, TM, TN, KSUB, DEPTH, NORM, KIND>),         \
                     dim3(wgs(16 * TM * WGM, 16 * TN * WGN)), dim3(64 * WGM * WGN), 0, st, ga)
  // (8-wave tiles need float32 A: row-major bf16 A rows do not split over 512 threads; a
  // stage of KSUB k-steps needs K % (32 KSUB) == 0, else one k-step per stage)
  const int ks = ga.K >> 5;
  const bool f = AIsFloat<TA>::value;
  switch ((f || tile < 4) && ks % 4 == 0 ? tile : 0) {
    case 1: MFMA_LAUNCH(2, 2, 2, 2, 2, 3); break;   //  64 x  64, 4 waves, BK  64
    case 2: MFMA_LAUNCH(2, 2, 2, 2, 4, 2); break;   //  64 x  64, 4 waves, BK 128
    case 3: MFMA_LAUNCH(2, 2, 2, 4, 2, 3); break;   //  64 x 128, 4 waves, BK  64
    case 4: if constexpr (AIsFloat<TA>::value) MFMA_LAUNCH(2, 4, 2, 4, 2, 2); break;  //  64 x 256, 8 waves
    case 5: if constexpr (AIsFloat<TA>::value && KIND != EPI_ARGMAX) MFMA_LAUNCH(2, 4, 4, 4, 2, 2); break;  // 128 x 256, 8 waves
    case 6: if constexpr (AIsFloat<TA>::value) MFMA_LAUNCH(2, 2, 4, 4, 2, 2); break;  // 128 x 128, 4 waves
    case 7: if constexpr (AIsFloat<TA>::value) MFMA_LAUNCH(2, 4, 2, 2, 4, 2); break;  //  64 x 128, 8 waves
    default:
      if (ks % 2) MFMA_LAUNCH(2, 2, 2, 2, 1, 3);
      else if (wgs(64, 128) >= num_cus()) MFMA_LAUNCH(2, 2, 2, 4, 2, 3);
      else MFMA_LAUNCH(2, 2, 2, 2, 2, 3);
  }
#undef MFMA_LAUNCH
  return hipGetLastError();
}

hipError_t launch_gemm(int dt, const GemmArgs& ga, hipStream_t st) {
  if (ga.M <= 0 || ga.N <= 0) return hipSuccess;
  const bool norm = ga.norm_g != nullptr;
  // the combinations the drafter / verifier use: normalised float32 A feeds QKV, gate/up,
  // the LM head and the injection K/V projection; plain float32 A feeds O and down; the
  // bf16 tapped features feed W_c
  if (ga.a_bf16) {
    if (norm || ga.e.kind != EPI_STORE_F32) return hipErrorInvalidValue;
    return launch_kind<bf16, false, EPI_STORE_F32>(dt, ga, st);
  }
  switch (ga.e.kind) {
    case EPI_QKV: return norm ? launch_kind<float, true, EPI_QKV>(dt, ga, st) : hipErrorInvalidValue;
    case EPI_SWIGLU: return norm ? launch_kind<float, true, EPI_SWIGLU>(dt, ga, st) : hipErrorInvalidValue;
    case EPI_ARGMAX: return norm ? launch_kind<float, true, EPI_ARGMAX>(dt, ga, st) : hipErrorInvalidValue;
    case EPI_INJECT_KV: return norm ? launch_kind<float, true, EPI_INJECT_KV>(dt, ga, st) : hipErrorInvalidValue;
    case EPI_RESID: return norm ? hipErrorInvalidValue : launch_kind<float, false, EPI_RESID>(dt, ga, st);
    case EPI_STORE_F32: return norm ? hipErrorInvalidValue : launch_kind<float, false, EPI_STORE_F32>(dt, ga, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dflash
