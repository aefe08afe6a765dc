// GEMM kernels: C[s][M][N] = A[M, K] x W^T with W [N, K] row-major (y = x W^T).
//
//  * gemm_skinny_bf16  (M <= 32): the weight-streaming shape of a drafter step at small
//    batch.  Each workgroup owns 16 output columns at a time and its waves split K; every
//    lane streams 16-byte slices of W rows straight into MFMA B fragments (no LDS), the
//    16x16 partial tiles of the waves are summed through LDS.  W is read exactly once.
//  * gemm_tiled_bf16   (M > 32): LDS-staged 128x128 tiles, 2x2 waves of 64x64, BK = 64,
//    global loads for the next K tile in flight while MFMAs consume the current one;
//    optional split-K into separate partial planes (summed by the consumer).
//  * gemm_f32          (float32 models): VALU 64x64 tiles, BK = 16.
//
// MFMA used: v_mfma_f32_16x16x32_bf16.  Operand layout (lane l, r = l % 16, g = l / 16):
// A fragment = A[r][8g .. 8g+7], B fragment = B[8g .. 8g+7][r] (i.e. W row r), and the
// accumulator holds D[4g + i][r], i = 0..3.
#include "common.h"
#include "kernels.h"

namespace dflash {

struct BSegDev {
  const bf16* ptr[8];
  int seg_rows, nseg, ldb;
  DF_DEV const bf16* row(int n) const {
    const int s = nseg > 1 ? n / seg_rows : 0;
    return ptr[s] + (size_t)(n - s * seg_rows) * ldb;
  }
};

// ---------------------------------------------------------------------------------------
template <int MT, int NW, int U>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_bf16(const bf16* __restrict__ A, int lda,
                                                            BSegDev B, float* __restrict__ C,
                                                            int M, int N, int K) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int KS = K >> 5;
  const int ks0 = (w * KS) / NW, ks1 = ((w + 1) * KS) / NW;
  const int n_tiles = (N + 15) >> 4;
  __shared__ f32x4 red[NW][MT][64];

  const bf16* arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + r, M - 1);
    arow[mt] = A + (size_t)m * lda + g * 8;
  }

  for (int t = blockIdx.x; t < n_tiles; t += gridDim.x) {
    const int n = min(t * 16 + r, N - 1);
    const bf16* wrow = B.row(n) + g * 8;
    f32x4 acc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    int ks = ks0;
    for (; ks + U <= ks1; ks += U) {
      bf16x8 wf[U];
      bf16x8 af[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u) wf[u] = *(const bf16x8*)(wrow + (size_t)(ks + u) * 32);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[u][mt] = *(const bf16x8*)(arow[mt] + (size_t)(ks + u) * 32);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][mt], wf[u], acc[mt], 0, 0, 0);
    }
    for (; ks < ks1; ++ks) {
      const bf16x8 wf = *(const bf16x8*)(wrow + (size_t)ks * 32);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 af = *(const bf16x8*)(arow[mt] + (size_t)ks * 32);
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wf, acc[mt], 0, 0, 0);
      }
    }

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) red[w][mt][lane] = acc[mt];
    __syncthreads();
    if (w < MT) {
      const int mt = w;
      f32x4 s = red[0][mt][lane];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) s += red[ww][mt][lane];
      const int col = t * 16 + r;
      if (col < N) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = mt * 16 + g * 4 + i;
          if (row < M) C[(size_t)row * N + col] = s[i];
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// 128 x 128 x 64 tiles, 256 threads (waves 2 x 2, 64 x 64 each).
#define TBM 128
#define TBN 128
#define TBK 64
#define TPAD 8

__global__ __launch_bounds__(256) void gemm_tiled_bf16(const bf16* __restrict__ A, int lda,
                                                       BSegDev B, float* __restrict__ C, int M,
                                                       int N, int K, int k_per_split) {
  __shared__ bf16 As[TBM][TBK + TPAD];
  __shared__ bf16 Bs[TBN][TBK + TPAD];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  const int n0 = blockIdx.x * TBN, m0 = blockIdx.y * TBM;
  const int s = blockIdx.z;
  const int kbeg = s * k_per_split, kend = min(K, kbeg + k_per_split);

  // global -> register staging: 4 x 16 B of A and of B per thread per K tile
  const bf16* ap[4];
  const bf16* bp[4];
  int lrow[4], lcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = tid + 256 * j;
    lrow[j] = c >> 3;
    lcol[j] = (c & 7) * 8;
    ap[j] = A + (size_t)min(m0 + lrow[j], M - 1) * lda + lcol[j];
    bp[j] = B.row(min(n0 + lrow[j], N - 1)) + lcol[j];
  }
  bf16x8 ra[4], rb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ra[j] = *(const bf16x8*)(ap[j] + kbeg);
    rb[j] = *(const bf16x8*)(bp[j] + kbeg);
  }

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg; k0 < kend; k0 += TBK) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *(bf16x8*)&As[lrow[j]][lcol[j]] = ra[j];
      *(bf16x8*)&Bs[lrow[j]][lcol[j]] = rb[j];
    }
    __syncthreads();
    if (k0 + TBK < kend) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        ra[j] = *(const bf16x8*)(ap[j] + k0 + TBK);
        rb[j] = *(const bf16x8*)(bp[j] + k0 + TBK);
      }
    }
#pragma unroll
    for (int kk = 0; kk < TBK; kk += 32) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)&As[wm * 64 + i * 16 + r][kk + g * 8];
#pragma unroll
      for (int j = 0; j < 4; ++j) bfr[j] = *(const bf16x8*)&Bs[wn * 64 + j * 16 + r][kk + g * 8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  float* Cs = C + (size_t)s * M * N;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + j * 16 + r;
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 64 + i * 16 + g * 4 + e;
        if (row < M) Cs[(size_t)row * N + col] = acc[i][j][e];
      }
    }
}

// ---------------------------------------------------------------------------------------
struct BSegF32 {
  const float* ptr[8];
  int seg_rows, nseg, ldb;
  DF_DEV const float* row(int n) const {
    const int s = nseg > 1 ? n / seg_rows : 0;
    return ptr[s] + (size_t)(n - s * seg_rows) * ldb;
  }
};

__global__ __launch_bounds__(256) void gemm_f32(const float* __restrict__ A, int lda, BSegF32 B,
                                                float* __restrict__ C, int M, int N, int K) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  const float* ap = A + (size_t)min(m0 + lr, M - 1) * lda + lk;
  const float* bp = B.row(min(n0 + lr, N - 1)) + lk;
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      As[lk + e][lr] = ap[k0 + e];
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + ty * 4 + i;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + tx * 4 + j;
      if (col < N) C[(size_t)row * N + col] = acc[i][j];
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

int gemm_splits(int dt, int M, int N, int K) {
  if (dt != BF16 || M <= 32) return 1;
  const int tiles = ((M + TBM - 1) / TBM) * ((N + TBN - 1) / TBN);
  int s = 1;
  // split K until the grid covers the chip twice, keeping >= 512 of K per split
  while (tiles * s < 512 && s < 4 && (K / (s * 2)) % TBK == 0 && K / (s * 2) >= 512) s *= 2;
  return s;
}

hipError_t launch_gemm(int dt, const void* A, int lda, const BSeg& B, float* C, int M, int N,
                       int K, int splits, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dt == F32) {
    BSegF32 b;
    for (int i = 0; i < 8; ++i) b.ptr[i] = (const float*)B.ptr[i];
    b.seg_rows = B.seg_rows;
    b.nseg = B.nseg;
    b.ldb = B.ldb;
    dim3 grid((N + 63) / 64, (M + 63) / 64);
    hipLaunchKernelGGL(gemm_f32, grid, dim3(256), 0, st, (const float*)A, lda, b, C, M, N, K);
    return hipGetLastError();
  }
  BSegDev b;
  for (int i = 0; i < 8; ++i) b.ptr[i] = (const bf16*)B.ptr[i];
  b.seg_rows = B.seg_rows;
  b.nseg = B.nseg;
  b.ldb = B.ldb;
  if (M <= 32) {
    const int n_tiles = (N + 15) / 16;
    const int grid = n_tiles < 8 * num_cus() ? n_tiles : 8 * num_cus();
    if (M <= 16)
      hipLaunchKernelGGL((gemm_skinny_bf16<1, 4, 8>), dim3(grid), dim3(256), 0, st,
                         (const bf16*)A, lda, b, C, M, N, K);
    else
      hipLaunchKernelGGL((gemm_skinny_bf16<2, 4, 8>), dim3(grid), dim3(256), 0, st,
                         (const bf16*)A, lda, b, C, M, N, K);
    return hipGetLastError();
  }
  const int kps = K / splits;
  dim3 grid((N + TBN - 1) / TBN, (M + TBM - 1) / TBM, splits);
  hipLaunchKernelGGL(gemm_tiled_bf16, grid, dim3(256), 0, st, (const bf16*)A, lda, b, C, M, N, K,
                     kps);
  return hipGetLastError();
}

}  // namespace dflash
