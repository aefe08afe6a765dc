// GEMM entry point and the float32-model kernel.  acc[m][n] = sum_k A[m][k] W[n][k]
// (y = x W^T), optional A-side RMSNorm, then one of the epilogues of epilogue.h.
//  * gemm_gemv_bf16 (gemv.hip, M <= 16): the weight-streaming shape of a drafter step.
//  * gemm_rows_bf16 (gemm_rows.hip, M > 16, few column tiles): row-resident K-split MFMA
//    GEMM + reduce; gemm_mfma_bf16 / gemm_wdirect_bf16 (gemm_mfma.hip, M > 16, many tiles).
//  * gemm_f32 (here, float32 models): VALU 64 x 64 tiles, BK = 16, row-major operands.
#include "gemm_common.h"

namespace dflash {

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
          k = umax64(k, pack_argmax_key(argmax_value(e, row, col0 + j, v[j]), col0 + j));
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

struct F32Launch {
  template <typename TA, bool NORM, int KIND>
  static hipError_t run(const GemmArgs& ga, hipStream_t st) {
    if constexpr (AIsFloat<TA>::value) {
      return launch1(gemm_f32<NORM, KIND>, dim3((ga.N + 63) / 64, (ga.M + 63) / 64), dim3(256), st, ga);
    } else {
      return hipErrorInvalidValue;
    }
  }
};

hipError_t launch_gemv(const GemmArgs& ga, hipStream_t st);
hipError_t launch_gemm_rows(const GemmArgs& ga, hipStream_t st);

hipError_t launch_gemm(int dt, const GemmArgs& ga, hipStream_t st) {
  if (ga.M <= 0 || ga.N <= 0) return hipSuccess;
  if (dt == F32) return dispatch_gemm<F32Launch>(ga, st);
  if (ga.M <= 16 && ga.K % (32 * GEMV_NW) == 0) return launch_gemv(ga, st);
  return launch_gemm_rows(ga, st);
}

}  // namespace dflash
