// Device helpers and host plumbing shared by the GEMM translation units (gemv.hip,
// gemm_mfma.hip, gemm.hip): B-operand addressing, the per-tile epilogue, the compensated
// A operand, and the dispatch over the operand / epilogue combinations in use.
//
// MFMA: v_mfma_f32_16x16x32_bf16.  Lane l (r = l % 16, g = l / 16) supplies A[r][8g..8g+7]
// and W row r's k-slice 8g..8g+7; the accumulator holds D[4g + i][r], i = 0..3.
#pragma once
#include "epilogue.h"

#define GEMV_NW 8    // waves per workgroup of the M <= 16 GEMV (K must be a multiple of 32 GEMV_NW)
#define GEMV_CH 16   // 32-wide steps per wave of its stationary-A form (K = 32 GEMV_NW GEMV_CH)

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

// one lane's 16 bytes of a weight fragment.  A launch reads every weight once: the loads
// carry the non-temporal hint (streamed, not kept in the caches), which measured faster on
// the M <= 16 GEMVs (LM head 205 -> 190 us, down 25.8 -> 23.8, QKV 18.7 -> 17.4).  Not for
// gate/up (epilogue kind SwiGLU): no faster there, and its HBM reads grew 15 % (FETCH_SIZE).
DF_DEV bf16x8 wload(const bf16* p) { return __builtin_nontemporal_load((const bf16x8*)p); }
template <int KIND>
DF_DEV bf16x8 wload_k(const bf16* p) {
  if constexpr (KIND == EPI_SWIGLU) return *(const bf16x8*)p;
  else return wload(p);
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

// the value whose maximum the argmax epilogue takes: the logit itself, or for sampling the
// tempered logit plus the row's Gumbel noise at this column
DF_DEV float argmax_value(const EpiArgs& e, int row, int col, float v) {
  if (!e.sample) return v;
  const int b = row / e.B, i = row - b * e.B;
  return v / e.temperature + gumbel_noise(e.seed, e.counter, 0, b, i, col);
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
      unsigned long long k = ok ? pack_argmax_key(argmax_value(e, row, col, v[i]), col) : 0ull;
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
// TA = pairf: the activations already split into (hi, lo) bf16 planes by pair_split.  Per
// 16-row block and 32-wide k-step the 2 KB of the float32 A-fragment layout hold the hi
// plane (lane l: 8 bf16 at byte 16 l) and then the lo plane, so a 4-byte pairf steps
// through the planes exactly as float32 steps through the fragments: the kernels address
// both alike and only skip the conversion (and the norm, folded in by pair_split).
struct pairf { float bits; };
template <> struct AIsFloat<pairf> { static constexpr bool value = true; };
template <typename TA> struct AIsPair { static constexpr bool value = false; };
template <> struct AIsPair<pairf> { static constexpr bool value = true; };

// v (8 raw A values) -> operand pair; with NORM, the sum of squares of the raw values is
// added to *ss and v is multiplied by the gain slice gv first.
template <bool NORM>
DF_DEV void a_operand(float v[8], const bf16x8 gv, float* ss, bf16x8& hi, bf16x8& lo) {
  if (NORM) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      *ss += v[e] * v[e];
      v[e] *= (float)gv[e];
    }
  }
  split8(v, hi, lo);
}


// ---------------------------------------------------------------------------------------
// Host side.
static inline int num_cus() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    hipDeviceProp_t p;
    n = (hipGetDeviceProperties(&p, dev) == hipSuccess && p.multiProcessorCount > 0) ? p.multiProcessorCount : 256;
  }
  return n;
}

// Launches kernel<<<grid, block, 0, st>>>(ga) and returns the launch status.
template <typename K>
static hipError_t launch1(K kernel, dim3 grid, dim3 block, hipStream_t st, const GemmArgs& ga) {
  hipLaunchKernelGGL(kernel, grid, block, 0, st, ga);
  return hipGetLastError();
}

// Calls F::run<TA, NORM, KIND>(ga, st) for the combinations the drafter and verifier use:
// normalised float32 A feeds QKV, gate/up, the LM head and the injection K/V projection;
// plain float32 A feeds O and down; the bf16 tapped features feed W_c.
template <typename F>
static hipError_t dispatch_gemm(const GemmArgs& ga, hipStream_t st) {
  const bool norm = ga.norm_g != nullptr;
  if (ga.a_pair) {
    if (norm || ga.a_bf16) return hipErrorInvalidValue;
    switch (ga.e.kind) {
      case EPI_QKV: return F::template run<pairf, false, EPI_QKV>(ga, st);
      case EPI_SWIGLU: return F::template run<pairf, false, EPI_SWIGLU>(ga, st);
      case EPI_ARGMAX: return F::template run<pairf, false, EPI_ARGMAX>(ga, st);
      case EPI_INJECT_KV: return F::template run<pairf, false, EPI_INJECT_KV>(ga, st);
      case EPI_RESID: return F::template run<pairf, false, EPI_RESID>(ga, st);
      case EPI_STORE_F32: return F::template run<pairf, false, EPI_STORE_F32>(ga, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (ga.a_bf16) {
    if (norm || ga.e.kind != EPI_STORE_F32) return hipErrorInvalidValue;
    return F::template run<bf16, false, EPI_STORE_F32>(ga, st);
  }
  switch (ga.e.kind) {
    case EPI_QKV: return norm ? F::template run<float, true, EPI_QKV>(ga, st)
                              : F::template run<float, false, EPI_QKV>(ga, st);
    case EPI_SWIGLU: return norm ? F::template run<float, true, EPI_SWIGLU>(ga, st)
                                 : F::template run<float, false, EPI_SWIGLU>(ga, st);
    case EPI_ARGMAX: return norm ? F::template run<float, true, EPI_ARGMAX>(ga, st) : hipErrorInvalidValue;
    case EPI_INJECT_KV: return norm ? F::template run<float, true, EPI_INJECT_KV>(ga, st) : hipErrorInvalidValue;
    case EPI_RESID: return norm ? hipErrorInvalidValue : F::template run<float, false, EPI_RESID>(ga, st);
    case EPI_STORE_F32: return norm ? F::template run<float, true, EPI_STORE_F32>(ga, st)
                                    : F::template run<float, false, EPI_STORE_F32>(ga, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dflash
