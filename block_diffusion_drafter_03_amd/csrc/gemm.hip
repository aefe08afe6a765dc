// GEMM kernels with fused epilogues: acc[m][n] = sum_k A[m][k] W[n][k] (y = x W^T),
// optional A-side RMSNorm, then one of the epilogues of epilogue.h.
//
// bfloat16 models: W in B-fragment order and float32 activations in A-fragment order
// (common.h), so every operand load of a wave is one contiguous 1 KB burst.  Activations
// enter the MFMAs as compensated (hi, lo) bf16 pairs; caller-supplied bf16 inputs (the
// tapped features of the fusion GEMM) are row-major and enter as they are.
//  * gemm_gemv_bf16   (M <= 16): the weight-streaming shape of a drafter step.  8 waves
//    split K, a workgroup walks 16-column tiles; see the kernel.
//  * gemm_tiled_bf16  (M > 16): 64x64 output tiles, 2x2 waves of 32x32, BK = 64, A and W
//    staged through LDS with the next K tile's global loads in flight during the MFMAs;
//    1-D grid remapped so that the M tiles sharing a W column block run on one XCD.
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

// ---------------------------------------------------------------------------------------
#define TB 64
#define TK 64
#define TPAD 8

// A tile (64 rows x 64 k) staging.  TA = float: 16 fragment halves of 1 KB (4 row blocks x
// 2 steps x 2 halves); thread c, slot j covers row 16 j + c % 16, k = 32 (c / 128) +
// 8 ((c % 64) / 16) + 4 ((c / 64) % 2) .. +3.  TA = bf16: row-major rows, 2 x 8 values.
template <typename TA> struct ATile;
template <> struct ATile<float> {
  static constexpr int SLOTS = 4, VALS = 4;
};
template <> struct ATile<bf16> {
  static constexpr int SLOTS = 2, VALS = 8;
};

template <typename TA, bool NORM, int KIND>
__global__ __launch_bounds__(256) void gemm_tiled_bf16(GemmArgs ga) {
  constexpr bool TWO = AIsFloat<TA>::value;
  constexpr int SLOTS = ATile<TA>::SLOTS, VALS = ATile<TA>::VALS;
  __shared__ __attribute__((aligned(16))) bf16 As[TWO ? 2 : 1][TB][TK + TPAD];
  __shared__ __attribute__((aligned(16))) bf16 Bs[TB][TK + TPAD];
  __shared__ float ss_part[NORM ? TB : 1][NORM ? 17 : 1];
  __shared__ float rstd_s[TB];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  const int M = ga.M, N = ga.N, K = ga.K, KS = K >> 5;
  const int MB = (M + 15) >> 4, NT = (N + 15) >> 4;
  const int mt_n = (M + TB - 1) / TB, nt_n = (N + TB - 1) / TB;
  const int T = mt_n * nt_n;
  // tiles ordered M-fastest; give each XCD (WG id mod 8) a contiguous run of tiles so the
  // M tiles that read the same W columns share an L2
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (blockIdx.x & 7) * (T >> 3) + (blockIdx.x >> 3);
  const int m0 = (t % mt_n) * TB, n0 = (t / mt_n) * TB;

  // ---- this thread's A slots ----
  int arow[SLOTS], acol[SLOTS];
  const TA* ap[SLOTS];
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) {
    if constexpr (TWO) {
      arow[j] = 16 * j + r;
      acol[j] = 32 * (tid >> 7) + 8 * g + 4 * ((tid >> 6) & 1);
      const int mb = min((m0 >> 4) + j, MB - 1);
      ap[j] = (const TA*)ga.A + ((size_t)(mb * KS + (tid >> 7)) * 2 + ((tid >> 6) & 1)) * 256 + lane * 4;
    } else {
      const int c = tid + 256 * j;
      arow[j] = c >> 3;
      acol[j] = (c & 7) * 8;
      ap[j] = (const TA*)ga.A + (size_t)min(m0 + arow[j], M - 1) * ga.lda + acol[j];
    }
  }
  // A slot loads of the K tile at k0 (float: the step advances by 2 per K tile)
  auto load_as = [&](int k0, float (*ra)[VALS]) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      if constexpr (TWO) {
        const float4 x = *(const float4*)(ap[j] + (size_t)(k0 >> 5) * 512);
        ra[j][0] = x.x; ra[j][1] = x.y; ra[j][2] = x.z; ra[j][3] = x.w;
      } else {
        load8(ap[j] + k0, ra[j]);
      }
    }
  };
  // ---- this thread's W slots: 2 x 16 B of the 8 fragment blocks of the tile ----
  const bf16* bp[2];
  int brow_[2], bcol[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int q = tid + 256 * j, blk = q >> 6, bl = q & 63;
    brow_[j] = 16 * (blk >> 1) + (bl & 15);
    bcol[j] = 32 * (blk & 1) + 8 * (bl >> 4);
    bp[j] = wblock(ga.B, min((n0 >> 4) + (blk >> 1), NT - 1), blk & 1, KS) + bl * 8;
  }
  const bf16* gk = NORM ? (const bf16*)ga.norm_g : nullptr;
  float ra[SLOTS][VALS];
  bf16x8 rb[2];
  float ss[SLOTS];
#pragma unroll
  for (int j = 0; j < SLOTS; ++j) ss[j] = 0.f;
  load_as(0, ra);
#pragma unroll
  for (int j = 0; j < 2; ++j) rb[j] = *(const bf16x8*)bp[j];
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
    for (int j = 0; j < SLOTS; ++j) {
      float v[8];
#pragma unroll
      for (int e = 0; e < VALS; ++e) {
        float x = ra[j][e];
        if (NORM) {
          ss[j] += x * x;
          x *= (float)gk[k0 + acol[j] + e];
        }
        v[e] = x;
      }
#pragma unroll
      for (int e = VALS; e < 8; ++e) v[e] = 0.f;
      bf16x8 hi, lo;
      split8(v, hi, lo);
      if constexpr (TWO) {
        bf16x4 h4 = {hi[0], hi[1], hi[2], hi[3]}, l4 = {lo[0], lo[1], lo[2], lo[3]};
        *(bf16x4*)&As[0][arow[j]][acol[j]] = h4;
        *(bf16x4*)&As[TWO ? 1 : 0][arow[j]][acol[j]] = l4;
      } else {
        *(bf16x8*)&As[0][arow[j]][acol[j]] = hi;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) *(bf16x8*)&Bs[brow_[j]][bcol[j]] = rb[j];
    __syncthreads();
    if (k0 + TK < K) {
      load_as(k0 + TK, ra);
#pragma unroll
      for (int j = 0; j < 2; ++j) rb[j] = *(const bf16x8*)(bp[j] + (size_t)((k0 + TK) >> 5) * 512);
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
    if constexpr (TWO) {
      // row 16 j + r collects its 16 contributors (tid / 16) in a fixed order
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) ss_part[arow[j]][tid >> 4] = ss[j];
      __syncthreads();
      if (tid < TB) {
        float s = 0.f;
        for (int i = 0; i < 16; ++i) s += ss_part[tid][i];
        rstd_s[tid] = 1.0f / sqrtf(s / (float)K + ga.eps);
      }
    } else {
      // the 8 threads loading one A row are consecutive lanes
#pragma unroll
      for (int j = 0; j < SLOTS; ++j) {
        float s = ss[j];
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        if ((tid & 7) == 0) rstd_s[arow[j]] = 1.0f / sqrtf(s / (float)K + ga.eps);
      }
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
