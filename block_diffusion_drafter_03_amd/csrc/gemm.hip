// GEMM entry point and the float32-model kernel.  acc[m][n] = sum_k A[m][k] W[n][k]
// (y = x W^T), optional A-side RMSNorm, then one of the epilogues of epilogue.h.
//  * gemm_gemv_bf16 (gemv.hip, M <= 16): the weight-streaming shape of a drafter step.
//  * gemm_rows_bf16 (gemm_rows.hip, M > 16, few column tiles): row-resident K-split MFMA
//    GEMM + reduce; gemm_mfma_bf16 / gemm_wdirect_bf16 (gemm_mfma.hip, M > 16, many tiles).
//  * gemm_f32 (here, float32 models): VALU 64 x 64 tiles, BK = 16, row-major operands.
//  * pair_split (here): for M > 16 the float32 activations are split into compensated
//    (hi, lo) bf16 planes once per GEMM, the A-side RMSNorm folded in, so that the MFMA
//    kernels load ready operands instead of converting them in every workgroup.
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
    if constexpr (AIsFloat<TA>::value && !AIsPair<TA>::value) {
      return launch1(gemm_f32<NORM, KIND>, dim3((ga.N + 63) / 64, (ga.M + 63) / 64), dim3(256), st, ga);
    } else {
      return hipErrorInvalidValue;
    }
  }
};

// ---------------------------------------------------------------------------------------
// Compensated operand planes of M float32 activation rows (A-fragment order, K = 32 KS):
// out holds, per 16-row block and k-step, the hi plane (1 KB: lane l = (r, g) has
// bf16(y[r][8g .. 8g+7])) followed by the lo plane (bf16 of y minus the hi value), with
// y = x (no norm) or y = x g / rms(x) (the RMSNorm of the GEMV epilogues, folded in; a
// row's sum of squares runs over the whole K in a fixed order).  A workgroup converts RW
// rows (16: a row block; 4 with the norm, whose statistics every workgroup gathers over the
// whole K for its own rows) over a chunk of `chunk` k-steps.  Grid: (row groups, chunks),
// 256 threads; rows past M in the last block are converted like the others (the GEMMs
// compute and discard them).
template <bool NORM>
__global__ __launch_bounds__(256) void pair_split(const float* A, int KS, const bf16* g, float eps,
                                                  int chunk, bf16* out) {
  constexpr int RW = NORM ? 4 : 16, PARTS = 256 / RW;
  const int tid = threadIdx.x;
  const int mb = blockIdx.x / (16 / RW), r0 = (blockIdx.x % (16 / RW)) * RW;
  const float* Ab = A + (size_t)mb * KS * 512;
  __shared__ float red[RW][PARTS + 1];
  __shared__ float rs[RW];
  if constexpr (NORM) {
    // thread (row r0 + rr, part p) sums the squares of its row over k-steps p, p + PARTS, ...
    const int rr = tid % RW, p = tid / RW;
    float s = 0.f;
    for (int ks = p; ks < KS; ks += PARTS) {
      const float* b = Ab + (size_t)ks * 512 + (r0 + rr) * 4;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 x = *(const float4*)(b + h * 256 + q * 64);
          s += x.x * x.x + x.y * x.y + x.z * x.z + x.w * x.w;
        }
    }
    red[rr][p] = s;
    __syncthreads();
    if (tid < RW) {
      float t = 0.f;
      for (int q = 0; q < PARTS; ++q) t += red[tid][q];
      rs[tid] = 1.0f / sqrtf(t / (float)(KS * 32) + eps);
    }
    __syncthreads();
  }
  // items: (k-step, lane of this workgroup's rows); 4 RW lanes per k-step
  const int ks0 = blockIdx.y * chunk, n = min(KS - ks0, chunk) * 4 * RW;
  for (int i = tid; i < n; i += 256) {
    const int ks = ks0 + i / (4 * RW), li = i % (4 * RW);
    const int lane = (li / RW) * 16 + r0 + li % RW;
    const float* b = Ab + (size_t)ks * 512 + lane * 4;
    const float4 x0 = *(const float4*)b, x1 = *(const float4*)(b + 256);
    float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    if constexpr (NORM) {
      const bf16x8 gv = *(const bf16x8*)(g + ks * 32 + (lane >> 4) * 8);
      const float rr = rs[li % RW];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = v[e] * (float)gv[e] * rr;
    }
    bf16x8 hi, lo;
    split8(v, hi, lo);
    bf16* o = out + ((size_t)mb * KS + ks) * 1024 + lane * 8;
    *(bf16x8*)o = hi;
    *(bf16x8*)(o + 512) = lo;
  }
}

size_t pair_plane_bytes(int rows, int max_k) { return (size_t)((rows + 15) / 16) * 16 * max_k * 4; }

hipError_t launch_gemv(const GemmArgs& ga, hipStream_t st);
hipError_t launch_gemm_rows(const GemmArgs& ga, hipStream_t st);

bool gemm_takes_gemv(int dt, const GemmArgs& ga) {
  return dt != F32 && !ga.a_pair && ga.M >= 1 && ga.M <= 16 && ga.K % (32 * GEMV_NW) == 0;
}

hipError_t launch_gemm(int dt, const GemmArgs& ga, hipStream_t st) {
  if (ga.M <= 0 || ga.N <= 0) return hipSuccess;
  if (ga.a_pair) {
    // the caller's activations are operand planes already (written so by their producer)
    if (dt == F32 || ga.M <= 16 || ga.norm_g || ga.a_bf16) return hipErrorInvalidValue;
    return launch_gemm_rows(ga, st);
  }
  if (dt == F32) return dispatch_gemm<F32Launch>(ga, st);
  if (gemm_takes_gemv(dt, ga)) return launch_gemv(ga, st);
  if (!ga.a_bf16 && ga.split.pair && pair_plane_bytes(ga.M, ga.K) <= ga.split.pair_bytes) {
    // about 256 workgroups over (row groups, K chunks)
    const int KS = ga.K / 32, groups = (ga.M + 15) / 16 * (ga.norm_g ? 4 : 1);
    int kc = (256 + groups - 1) / groups;
    if (kc > KS) kc = KS;
    const int chunk = (KS + kc - 1) / kc;
    const dim3 grid(groups, (KS + chunk - 1) / chunk);
    if (ga.norm_g)
      hipLaunchKernelGGL(pair_split<true>, grid, dim3(256), 0, st, (const float*)ga.A, KS,
                         (const bf16*)ga.norm_g, ga.eps, chunk, (bf16*)ga.split.pair);
    else
      hipLaunchKernelGGL(pair_split<false>, grid, dim3(256), 0, st, (const float*)ga.A, KS, nullptr,
                         ga.eps, chunk, (bf16*)ga.split.pair);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    GemmArgs gp = ga;
    gp.A = ga.split.pair;
    gp.a_pair = 1;
    gp.norm_g = nullptr;
    return launch_gemm_rows(gp, st);
  }
  return launch_gemm_rows(ga, st);
}

}  // namespace dflash
