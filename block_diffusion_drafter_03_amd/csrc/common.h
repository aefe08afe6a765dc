// Shared device helpers for libdflash's gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

#define DF_DEV __device__ __forceinline__

DF_DEV float to_f(float x) { return x; }
DF_DEV float to_f(bf16 x) { return (float)x; }
template <typename T> DF_DEV T from_f(float x);
template <> DF_DEV float from_f<float>(float x) { return x; }
template <> DF_DEV bf16 from_f<bf16>(float x) { return (bf16)x; }

// Compensated bf16 operands.  Activations live in float32; a bf16 MFMA that takes one as
// an operand takes it as the pair hi = bf16(x) (nearest), lo = bf16(x - hi), which holds x
// to ~2^-17 relative.  Against a bf16 operand w both products are exact and the MFMA
// accumulates in float32, so hi*w + lo*w carries float32-class accuracy at the cost of a
// second MFMA on the same fragment (spare issue slots in the bandwidth-bound kernels).
DF_DEV void split8(const float v[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const bf16 h = (bf16)v[e];
    hi[e] = h;
    lo[e] = (bf16)(v[e] - (float)h);
  }
}
DF_DEV void load8(const float* p, float v[8]) {
  const float4 x0 = *(const float4*)p, x1 = *(const float4*)(p + 4);
  v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
  v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
}
DF_DEV void load8(const bf16* p, float v[8]) {
  const bf16x8 x = *(const bf16x8*)p;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)x[e];
}

// ---- MFMA-fragment layouts in HBM (bfloat16 models) ----
// A v_mfma_f32_16x16x32_bf16 operand covers 16 rows x 32 k as 64 lanes x 8 values: lane
// l = 16 g + r holds row r, k = 8g .. 8g+7.  Data that feeds such operands is stored in
// that order, so every wave-wide 16-byte load reads 1 KB contiguous.
//  * bf16 weights W [N, K] (N padded to a multiple of 16): one 1 KB block per (16-row tile
//    t, 32-wide step s), blocks ordered (t, s), lanes in order inside a block.
//  * float32 activations A [M, K] (M padded to a multiple of 16): per (16-row block, step)
//    two 1 KB halves, the first holding k % 8 < 4 of every lane, the second k % 8 >= 4.
DF_DEV size_t wfrag_off(int n, int k, int KS) {
  return ((size_t)((n >> 4) * KS + (k >> 5)) * 64 + ((k & 31) >> 3) * 16 + (n & 15)) * 8 + (k & 7);
}
DF_DEV size_t afrag_off(int m, int k, int KS) {
  return ((size_t)(((m >> 4) * KS + (k >> 5)) * 2 + ((k & 7) >> 2))) * 256 +
         (((k & 31) >> 3) * 16 + (m & 15)) * 4 + (k & 3);
}
//  * the same activations as compensated operand planes (bf16, the M > 16 GEMMs' input):
//    per (16-row block, step) 2 KB, the hi plane (lane (m % 16) + 16 ((k % 32) / 8) holding
//    8 consecutive k) then the lo plane 512 elements further.  pfrag_off is the hi element.
DF_DEV size_t pfrag_off(int m, int k, int KS) {
  return ((size_t)((m >> 4) * KS + (k >> 5))) * 1024 + (((k & 31) >> 3) * 16 + (m & 15)) * 8 + (k & 7);
}
// v as a (hi, lo) bf16 pair in the planes at hi element p
DF_DEV void store_pair(bf16* planes, size_t p, float v) {
  const bf16 h = (bf16)v;
  planes[p] = h;
  planes[p + 512] = (bf16)(v - (float)h);
}

// Entry i (< 8) of a small pointer table held in a kernel argument, by unrolled selects:
// a dynamically indexed private array would be placed in scratch memory.
template <typename P>
DF_DEV P pick8(P const (&t)[8], int i) {
  P p = t[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) p = i == j ? t[j] : p;
  return p;
}

// Wave64 reductions (xor butterflies over all 64 lanes).
DF_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DF_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Sum over a workgroup of up to 1024 threads; `red` must hold >= 16 floats.  All threads
// receive the total.  Deterministic: a fixed butterfly then a fixed-order sum.
DF_DEV float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// RoPE angle for position p and pair index i of a head of width d, evaluated in float64
// and rounded to float32 (cos, sin).
DF_DEV void rope_cs(int64_t p, int i, int d, double base, float* c, float* s) {
  const double theta = pow(base, -2.0 * (double)i / (double)d);
  const double a = (double)p * theta;
  *c = (float)cos(a);
  *s = (float)sin(a);
}

// Counter-based uniforms for sampling: draw number index + 1 of a splitmix64 stream seeded
// with `seed` (Vigna's published mixing function over the Weyl sequence of step
// 0x9E3779B97F4A7C15), index = (((counter * 4 + purpose) * 4096 + b) * 128 + i) * 262144 + v,
// keeping the top 23 bits: u = (r >> 41) + 1/2, over 2^23 - exact in float32 and strictly
// inside (0, 1).  Purposes: 0 drafter noise (b, position i, id v), 1 acceptance uniforms
// (b, position i, v = 0), 2 noise of the emitted token (b, target row i, id v).
DF_DEV float rng_uniform(unsigned long long seed, unsigned counter, unsigned purpose, unsigned b,
                         unsigned i, unsigned v) {
  const unsigned long long idx =
      ((((unsigned long long)counter * 4ull + purpose) * 4096ull + b) * 128ull + i) * 262144ull + v;
  unsigned long long z = seed + (idx + 1ull) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return ((float)(unsigned)(z >> 41) + 0.5f) * 1.1920928955078125e-7f;   // 2^-23
}
// Gumbel noise -log(-log(u)): argmax(x + noise) samples softmax(x)
DF_DEV float gumbel_noise(unsigned long long seed, unsigned counter, unsigned purpose, unsigned b,
                          unsigned i, unsigned v) {
  return -logf(-logf(rng_uniform(seed, counter, purpose, b, i, v)));
}

// Device error bits (mirror of DFLASH_DEVERR_*).
#define DEVERR_PAGE 1
#define DEVERR_TOKEN 2
#define DEVERR_TAU 4
DF_DEV void flag_error(int32_t* flags, int bit) {
  if (flags) atomicOr(flags, bit);
}
