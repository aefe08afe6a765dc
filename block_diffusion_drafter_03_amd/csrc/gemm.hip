// GEMM kernels with fused epilogues: acc[m][n] = sum_k A[m][k] W[n][k] (y = x W^T, W row-major
// [N, K]), optional A-side RMSNorm, then one of the epilogues of epilogue.h.
//
//  * gemm_skinny_bf16  (M <= 32): the weight-streaming shape of a drafter step at small
//    batch.  A workgroup owns 16 output columns at a time and its 4 waves split K; each
//    lane streams 16-byte slices of W rows straight into MFMA B fragments (no LDS), and the
//    waves' 16x16 partial tiles are summed through LDS.  W is read exactly once.
//  * gemm_tiled_bf16   (M > 32): 64x64 output tiles, 2x2 waves of 32x32, BK = 64, A and W
//    tiles staged through LDS with the next K tile's global loads in flight during the
//    MFMAs; 1-D grid remapped so that the M tiles sharing a W column block run on the same
//    XCD (one L2) back to back.
//  * gemm_f32          (float32 models): VALU 64x64 tiles, BK = 16.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l (r = l % 16, g = l / 16) supplies A[r][8g..8g+7]
// and W row r's k-slice 8g..8g+7; the accumulator holds D[4g + i][r], i = 0..3.
#include "epilogue.h"

namespace dflash {

// Row n of the B operand (W rows, possibly split into equal segments at different
// addresses), read straight from the kernel argument.
template <typename T>
DF_DEV const T* brow(const BSeg& b, int n) {
  const int s = b.nseg > 1 ? n / b.seg_rows : 0;
  return (const T*)pick8(b.ptr, s) + (size_t)(n - s * b.seg_rows) * b.ldb;
}

// A row m of the GEMM -> row of the A buffer (skipping the anchor row of each block when
// only the masked rows of the drafter feed the LM head).
DF_DEV int a_row_index(int m, int skipB) { return skipB ? m + m / (skipB - 1) + 1 : m; }

DF_DEV unsigned long long shfl_xor_u64(unsigned long long v, int mask) {
  const unsigned lo = __shfl_xor((unsigned)(v & 0xFFFFFFFFull), mask, 64);
  const unsigned hi = __shfl_xor((unsigned)(v >> 32), mask, 64);
  return ((unsigned long long)hi << 32) | lo;
}
DF_DEV unsigned long long umax64(unsigned long long a, unsigned long long b) { return a > b ? a : b; }


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
      if (ok && e.logits) e.logits[(size_t)row * N + col] = v[i];
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
// A operand helpers.  TA = float: activations, taken as a compensated (hi, lo) bf16 pair
// (two MFMAs per W fragment); TA = bf16: inputs already in bf16 (one MFMA).
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

// ---------------------------------------------------------------------------------------
// 16 < M <= 32 (and M <= 16 with few output tiles): 4 waves split K; A and W fragments are
// both loaded per 32-wide K step.
template <typename TA, int MT, int NW, int U, bool NORM, int KIND>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_bf16(GemmArgs ga) {
  constexpr bool TWO = AIsFloat<TA>::value;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int M = ga.M, N = ga.N, K = ga.K;
  const int KS = K >> 5;
  const int ks0 = (w * KS) / NW, ks1 = ((w + 1) * KS) / NW;
  const int n_tiles = (N + 15) >> 4;
  __shared__ f32x4 red[NW][MT][64];
  __shared__ float ss_red[NW][MT * 16];
  __shared__ float rstd[MT * 16];

  const TA* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r, M - 1);
    arow[mt] = (const TA*)ga.A + (size_t)a_row_index(m, ga.a_skip_B) * ga.lda + g * 8;
  }
  const bf16* gk = NORM ? (const bf16*)ga.norm_g + g * 8 : nullptr;
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};
  bool first = true;

  for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int n = min(t * 16 + r, N - 1);
    const bf16* wrow = brow<bf16>(ga.B, n) + g * 8;
    f32x4 acc[MT];
    float ss[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      ss[mt] = 0.f;
    }
    for (int ks = ks0; ks < ks1; ks += U) {
      bf16x8 wf[U];
      float av[U][MT][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int k = min(ks + u, ks1 - 1);
        wf[u] = *(const bf16x8*)(wrow + (size_t)k * 32);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) load8(arow[mt] + (size_t)k * 32, av[u][mt]);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ks + u >= ks1) break;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          bf16x8 hi, lo;
          if (first)
            a_operand<NORM, true>(av[u][mt], gk + (size_t)(ks + u) * 32, &ss[mt], hi, lo);
          else
            a_operand<NORM, false>(av[u][mt], gk + (size_t)(ks + u) * 32, &ss[mt], hi, lo);
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, wf[u], acc[mt], 0, 0, 0);
          if (TWO) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, wf[u], acc[mt], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[w][mt][lane] = acc[mt];
    if (NORM && first) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float s = ss[mt] + __shfl_xor(ss[mt], 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (g == 0) ss_red[w][mt * 16 + r] = s;
      }
    }
    __syncthreads();
    if (NORM && first) {
      if (threadIdx.x < MT * 16) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += ss_red[ww][threadIdx.x];
        rstd[threadIdx.x] = 1.0f / sqrtf(s / (float)K + ga.eps);
      }
      __syncthreads();
    }
    first = false;
    if (w < MT) {
      const int mt = w;
      f32x4 s = red[0][mt][lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) s += red[ww][mt][lane];
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = NORM ? s[i] * rstd[mt * 16 + g * 4 + i] : s[i];
      tile_epilogue<bf16, KIND>(ga, mt * 16 + g * 4, t * 16 + r, v, r, best);
    }
    __syncthreads();
  }
  if (KIND == EPI_ARGMAX && w < MT && r == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = w * 16 + g * 4 + i;
      if (row < M && best[i]) atomicMax(&ga.e.keys[row], best[i]);
    }
  }
}

// M <= 16: NW waves split K, one 32-wide step per MFMA (pair).  With ASTAT each wave keeps
// its K-slice of the A rows for all of the workgroup's tiles, already multiplied by the
// RMSNorm gain and split into (hi, lo) (rstd is applied in the epilogue): hi in registers,
// lo in LDS (128 KB: one workgroup owns the CU), so the vector memory path carries only W:
// a wave issues all of its W loads of a tile at once (CH steps, 1 KB each) and the CU keeps
// 128 KB in flight.  Without ASTAT (K > 4096) A and W are streamed together in chunks of
// CHS steps.  8 waves of 512 threads leave each wave 256 registers, so the stationary A,
// a full tile of W in flight and the epilogue never spill.
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
  const int spw = (K >> 5) / NW;                 // K % (32 NW) == 0
  const int ks0 = w * spw;
  const int n_tiles = (N + 15) >> 4;
  __shared__ f32x4 red[NW][64];
  __shared__ f32x4 done[GEMV_MAX_TILES][64];
  __shared__ float ss_red[NW][16];
  __shared__ float rstd[16];
  __shared__ bf16x8 alo[ASTAT && TWO ? NW : 1][ASTAT && TWO ? CH : 1][64];
  // running argmax keys of wave 0's lanes (kept out of the main loop's registers)
  __shared__ unsigned long long bsh[KIND == EPI_ARGMAX ? 4 : 1][64];
  const TA* arow = (const TA*)ga.A + (size_t)a_row_index(min(r, M - 1), ga.a_skip_B) * ga.lda + g * 8;
  const bf16* gk = NORM ? (const bf16*)ga.norm_g + g * 8 : nullptr;
  int nbuf = 0;
  if (KIND == EPI_ARGMAX && w == 0)
#pragma unroll
    for (int i = 0; i < (KIND == EPI_ARGMAX ? 4 : 1); ++i) bsh[i][lane] = 0ull;

  bf16x8 ah[ASTAT ? CH : 1];
  // W loads of this workgroup's first tile go out before the A prologue (independent)
  bf16x8 wn[CH];
  auto load_w = [&](int t) {
    const bf16* wrow = brow<bf16>(ga.B, min(t * 16 + r, N - 1)) + g * 8;
#pragma unroll
    for (int s = 0; s < CH; ++s)
      if (s < spw) wn[s] = *(const bf16x8*)(wrow + (size_t)(ks0 + s) * 32);
  };
  if constexpr (ASTAT) {
    if (blockIdx.x < n_tiles) load_w(blockIdx.x);
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < CH; ++s) {
      if (s < spw) {
        float v[8];
        load8(arow + (size_t)(ks0 + s) * 32, v);
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
      const bf16* wrow = brow<bf16>(ga.B, min(t * 16 + r, N - 1)) + g * 8;
      for (int c0 = 0; c0 < spw; c0 += CHS) {
        bf16x8 wf[CHS];
        float av[CHS][8];
#pragma unroll
        for (int s = 0; s < CHS; ++s) {
          const int k = ks0 + min(c0 + s, spw - 1);
          wf[s] = *(const bf16x8*)(wrow + (size_t)k * 32);
          load8(arow + (size_t)k * 32, av[s]);
        }
#pragma unroll
        for (int s = 0; s < CHS; ++s)
          if (c0 + s < spw) {
            bf16x8 hi, lo;
            split8(av[s], hi, lo);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, wf[s], acc, 0, 0, 0);
            if constexpr (TWO) acc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, wf[s], acc2, 0, 0, 0);
          }
      }
    }
    red[w][lane] = acc + acc2;
    __syncthreads();
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

// Variant selection for M <= 16 (benchmark sweeps may force one with DFLASH_GEMV=1..2):
// 1 = 4-wave split-K (gemm_skinny_bf16), 2 = gemm_gemv_bf16 (default where it fits).
static int gemv_variant() {
  static int v = -1;
  if (v < 0) {
    const char* s = getenv("DFLASH_GEMV");
    v = s && *s ? atoi(s) : 0;
  }
  return v;
}

// ---------------------------------------------------------------------------------------
#define TB 64
#define TK 64
#define TPAD 8

template <typename TA, bool NORM, int KIND>
__global__ __launch_bounds__(256) void gemm_tiled_bf16(GemmArgs ga) {
  constexpr bool TWO = AIsFloat<TA>::value;
  __shared__ __attribute__((aligned(16))) bf16 As[TWO ? 2 : 1][TB][TK + TPAD];
  __shared__ __attribute__((aligned(16))) bf16 Bs[TB][TK + TPAD];
  __shared__ float rstd_s[TB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  const int M = ga.M, N = ga.N, K = ga.K;
  const int mt_n = (M + TB - 1) / TB, nt_n = (N + TB - 1) / TB;
  const int T = mt_n * nt_n;
  // tiles ordered M-fastest; give each XCD (WG id mod 8) a contiguous run of tiles so the
  // M tiles that read the same W columns share an L2
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int m0 = (t % mt_n) * TB, n0 = (t / mt_n) * TB;

  const TA* ap[2];
  const bf16* bp[2];
  int lrow[2], lcol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + 256 * j;
    lrow[j] = c >> 3;
    lcol[j] = (c & 7) * 8;
    ap[j] = (const TA*)ga.A + (size_t)a_row_index(min(m0 + lrow[j], M - 1), ga.a_skip_B) * ga.lda + lcol[j];
    bp[j] = brow<bf16>(ga.B, min(n0 + lrow[j], N - 1)) + lcol[j];
  }
  const bf16* gk = NORM ? (const bf16*)ga.norm_g : nullptr;
  float ra[2][8];
  bf16x8 rb[2];
  float ss[2] = {0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    load8(ap[j], ra[j]);
    rb[j] = *(const bf16x8*)(bp[j]);
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 hi, lo;
      a_operand<NORM, true>(ra[j], gk + k0 + lcol[j], &ss[j], hi, lo);
      *(bf16x8*)&As[0][lrow[j]][lcol[j]] = hi;
      if constexpr (TWO) *(bf16x8*)&As[TWO ? 1 : 0][lrow[j]][lcol[j]] = lo;
      *(bf16x8*)&Bs[lrow[j]][lcol[j]] = rb[j];
    }
    __syncthreads();
    if (k0 + TK < K) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        load8(ap[j] + k0 + TK, ra[j]);
        rb[j] = *(const bf16x8*)(bp[j] + k0 + TK);
      }
    }
#pragma unroll
    for (int kk = 0; kk < TK; kk += 32) {
      bf16x8 bfr[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = *(const bf16x8*)&Bs[wn * 32 + j * 16 + r][kk + g * 8];
#pragma unroll
      for (int p = 0; p < (TWO ? 2 : 1); ++p) {
        bf16x8 af[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8*)&As[p][wm * 32 + i * 16 + r][kk + g * 8];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (NORM) {
    // the 8 threads loading one A row are consecutive lanes
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float s = ss[j];
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      s += __shfl_xor(s, 4, 64);
      if ((tid & 7) == 0) rstd_s[lrow[j]] = 1.0f / sqrtf(s / (float)K + ga.eps);
    }
    __syncthreads();
  }
  unsigned long long best[2][4] = {{0ull, 0ull, 0ull, 0ull}, {0ull, 0ull, 0ull, 0ull}};
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int lr0 = wm * 32 + i * 16 + g * 4;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = NORM ? acc[i][j][e] * rstd_s[lr0 + e] : acc[i][j][e];
      tile_epilogue<bf16, KIND>(ga, m0 + lr0, n0 + wn * 32 + j * 16 + r, v, r, best[i]);
    }
  if (KIND == EPI_ARGMAX && r == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 32 + i * 16 + g * 4 + e;
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
  const float* ap = (const float*)ga.A + (size_t)a_row_index(min(m0 + lr, M - 1), ga.a_skip_B) * ga.lda + lk;
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
          if (e.logits) e.logits[(size_t)row * N + col0 + j] = v[j];
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
  if (M <= 16) {
    int v = gemv_variant();
    const bool fits = ga.K % (32 * GEMV_NW) == 0 && !(NORM && ga.K > 4096);
    if (v < 1 || v > 2 || !fits) v = fits ? 2 : 1;
    if (v == 2) {
      // one workgroup per CU (the stationary A's LDS) walking the tiles; the deferred
      // epilogue buffer bounds the tiles per workgroup
      int grid = n_tiles < num_cus() ? n_tiles : num_cus();
      if (KIND != EPI_ARGMAX && grid * GEMV_MAX_TILES < n_tiles)
        grid = (n_tiles + GEMV_MAX_TILES - 1) / GEMV_MAX_TILES;
      if (ga.K <= 4096)
        hipLaunchKernelGGL((gemm_gemv_bf16<TA, GEMV_NW, NORM, true, KIND>), dim3(grid), dim3(GEMV_NW * 64), 0, st, ga);
      else
        hipLaunchKernelGGL((gemm_gemv_bf16<TA, GEMV_NW, false, false, KIND>), dim3(grid), dim3(GEMV_NW * 64), 0, st, ga);
      return hipGetLastError();
    }
  }
  if (M <= 32) {
    const int grid = n_tiles < 8 * num_cus() ? n_tiles : 8 * num_cus();
    if (M <= 16)
      hipLaunchKernelGGL((gemm_skinny_bf16<TA, 1, 4, 8, NORM, KIND>), dim3(grid), dim3(256), 0, st, ga);
    else
      hipLaunchKernelGGL((gemm_skinny_bf16<TA, 2, 4, 4, NORM, KIND>), dim3(grid), dim3(256), 0, st, ga);
    return hipGetLastError();
  }
  const int tiles = ((M + TB - 1) / TB) * ((N + TB - 1) / TB);
  hipLaunchKernelGGL((gemm_tiled_bf16<TA, NORM, KIND>), dim3(tiles), dim3(256), 0, st, ga);
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
